// Grouped output projection ([V4-CN] "DeepSeek-V4中文翻译" §2.3.1: the n_h core-attention
// outputs of a token are split into g groups, each projected to a d_g-dim intermediate
// output, and the intermediates are projected to the model dim d; §4.2.1 gives g = 16,
// d_g = 1024, d = 7168 for V4-Pro).  Two launches of one bf16 GEMM:
//   mid[t, j d_g + i] = sum_k o[t, j K + k] w_group[j, i, k]   (K = (n_h / g) c; batch j)
//   out[t, i]        = sum_k mid[t, k] w_out[i, k]            (K = g d_g)
// Weights are [out, in] matrices, so both operands of C = A W^T are contiguous along
// the contraction and load straight into the MFMA operand layout: lane (col, grp)
// holds 8 consecutive k of row col (v_mfma_f32_16x16x32_bf16, fp32 accumulation).
//
// Each wave computes a 16 x 64 block of C (four 16 x 16 MFMA accumulators) over its
// range of the contraction, its operands loaded from global memory two k-steps ahead
// of the products.  A workgroup of four waves covers WM x 16 rows and WN x 64 columns
// (WM WN = 4): a few rows (decode) take 16 x 256 tiles, so every weight row is read by
// one wave only and the weights stream from HBM once; many rows take 64 x 64 tiles,
// whose four waves share each weight fragment through the L1 cache.  With a few rows
// the tiles alone cannot fill the chip, so the contraction is split over workgroups:
// each writes an fp32 partial tile and a second pass sums the partials in split order
// (deterministic), converting to the output format.
#include "device_common.h"
#include "launch.h"

#include <algorithm>

namespace csa {

namespace {

struct GemmArgs {
  const uint16_t* A;  // [batch][M, K] rows at stride lda, batch stride sa
  const uint16_t* W;  // [batch][N, K] rows at stride K, batch stride sw
  void* C;            // [batch][M, N] rows at stride ldc, batch stride sc
  int64_t M, N, K, lda, ldc, sa, sw, sc;
  int out_f32;
  int64_t batch;
  int ksplit;         // contraction split over workgroups (1: no split)
  int steps_per_split;
  float* part;        // ksplit > 1: fp32 partials [ksplit][batch][M][N]
};

constexpr int kKStep = 32;
constexpr int kAhead = 2;  // k-steps loaded ahead of the products
constexpr int kFewRows = 32;          // at most this many rows: 16 x 256 tiles
constexpr int kTargetGroups = 1024;   // workgroups a split launch aims for
constexpr int kMinSplitSteps = 8;     // k-steps per split at least

template <int WM, int WN>
__global__ __launch_bounds__(256) void gemm_bf16_kernel(GemmArgs a) {
  static_assert(WM * WN == 4, "four waves");
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int64_t batch = blockIdx.z / a.ksplit;
  const int split = blockIdx.z % a.ksplit;
  const int64_t m0 = (static_cast<int64_t>(blockIdx.y) * WM + wid / WN) * 16;
  const int64_t n0 = (static_cast<int64_t>(blockIdx.x) * WN + wid % WN) * 64;
  if (m0 >= a.M || n0 >= a.N) return;  // a whole wave outside C (no barrier below)
  // operand rows, clamped into C's extent (rows past it are computed and not stored)
  const int64_t am = min(m0 + col, a.M - 1);
  const uint16_t* ap = a.A + batch * a.sa + am * a.lda + 8 * grp;
  const uint16_t* wp[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    wp[nb] = a.W + batch * a.sw + min(n0 + 16 * nb + col, a.N - 1) * a.K + 8 * grp;
  const int s_begin = split * a.steps_per_split;
  const int nsteps = min(static_cast<int>(a.K / kKStep) - s_begin, a.steps_per_split);
  ap += static_cast<int64_t>(s_begin) * kKStep;
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) wp[nb] += static_cast<int64_t>(s_begin) * kKStep;

  f32x4 acc[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 af[kAhead + 1], wf[kAhead + 1][4];
  auto load = [&](int slot, int s) {
    af[slot] = *reinterpret_cast<const bf16x8*>(ap + static_cast<int64_t>(s) * kKStep);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) wf[slot][nb] = *reinterpret_cast<const bf16x8*>(wp[nb] + static_cast<int64_t>(s) * kKStep);
  };
#pragma unroll
  for (int s = 0; s < kAhead; ++s)
    if (s < nsteps) load(s, s);
  for (int s0 = 0; s0 < nsteps; s0 += kAhead + 1) {
#pragma unroll
    for (int u = 0; u <= kAhead; ++u) {
      const int s = s0 + u;
      if (s >= nsteps) break;
      if (s + kAhead < nsteps) load((u + kAhead) % (kAhead + 1), s + kAhead);
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[u], wf[u][nb], acc[nb], 0, 0, 0);
    }
  }
  // lane (col, grp) holds C[m0 + 4 grp + r][n0 + 16 nb + col]
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int64_t n = n0 + 16 * nb + col;
    if (n >= a.N) continue;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t m = m0 + 4 * grp + r;
      if (m >= a.M) continue;
      if (a.ksplit > 1) {
        a.part[((split * a.batch + batch) * a.M + m) * a.N + n] = acc[nb][r];
        continue;
      }
      const int64_t o = batch * a.sc + m * a.ldc + n;
      if (a.out_f32) static_cast<float*>(a.C)[o] = acc[nb][r];
      else static_cast<uint16_t*>(a.C)[o] = f32_to_bf16(acc[nb][r]);
    }
  }
}

// Few rows (decode): a wave computes every row (MB 16-row blocks) of 64 columns, so
// each weight row is read by one wave only.  A lane loads 32 contiguous bytes of its
// row per 64-element step (4 lanes: one 128-byte line), which feed two MFMAs: both
// operands take the same permutation of the contraction index (lane group g holds
// elements 16 g .. 16 g + 15 of the step; the first MFMA takes the first 8 of them,
// the second the rest), so the products sum over the same elements.  Two steps of
// loads are kept in flight ahead of the products.
constexpr int kFewStep = 64;
constexpr int kFewAhead = 2;

template <int MB>
__global__ __launch_bounds__(256) void gemm_few_kernel(GemmArgs a) {
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x >> 6));
  const int col = lane & 15;
  const int grp = lane >> 4;
  const int64_t batch = blockIdx.z / a.ksplit;
  const int split = blockIdx.z % a.ksplit;
  const int64_t n0 = (static_cast<int64_t>(blockIdx.x) * 4 + wid) * 64;
  if (n0 >= a.N) return;  // a whole wave outside C (no barrier below)
  const int s_begin = split * a.steps_per_split;
  const int nsteps = min(static_cast<int>(a.K / kFewStep) - s_begin, a.steps_per_split);
  const uint16_t* ap[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    ap[mb] = a.A + batch * a.sa + min(static_cast<int64_t>(16 * mb + col), a.M - 1) * a.lda + 16 * grp +
             static_cast<int64_t>(s_begin) * kFewStep;
  const uint16_t* wp[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
    wp[nb] = a.W + batch * a.sw + min(n0 + 16 * nb + col, a.N - 1) * a.K + 16 * grp +
             static_cast<int64_t>(s_begin) * kFewStep;

  f32x4 acc[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4{0.f, 0.f, 0.f, 0.f};
  bf16x8 af[kFewAhead + 1][MB][2], wf[kFewAhead + 1][4][2];
  auto load = [&](int slot, int s) {
    const int64_t o = static_cast<int64_t>(s) * kFewStep;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      af[slot][mb][0] = *reinterpret_cast<const bf16x8*>(ap[mb] + o);
      af[slot][mb][1] = *reinterpret_cast<const bf16x8*>(ap[mb] + o + 8);
    }
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      wf[slot][nb][0] = *reinterpret_cast<const bf16x8*>(wp[nb] + o);
      wf[slot][nb][1] = *reinterpret_cast<const bf16x8*>(wp[nb] + o + 8);
    }
  };
#pragma unroll
  for (int s = 0; s < kFewAhead; ++s)
    if (s < nsteps) load(s, s);
  for (int s0 = 0; s0 < nsteps; s0 += kFewAhead + 1) {
#pragma unroll
    for (int u = 0; u <= kFewAhead; ++u) {
      const int s = s0 + u;
      if (s >= nsteps) break;
      if (s + kFewAhead < nsteps) load((u + kFewAhead) % (kFewAhead + 1), s + kFewAhead);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int nb = 0; nb < 4; ++nb)
            acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[u][mb][h], wf[u][nb][h], acc[mb][nb], 0, 0, 0);
    }
  }
  // lane (col, grp) holds C[16 mb + 4 grp + r][n0 + 16 nb + col]
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int64_t n = n0 + 16 * nb + col;
      if (n >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = 16 * mb + 4 * grp + r;
        if (m >= a.M) continue;
        if (a.ksplit > 1) {
          a.part[((split * a.batch + batch) * a.M + m) * a.N + n] = acc[mb][nb][r];
          continue;
        }
        const int64_t o = batch * a.sc + m * a.ldc + n;
        if (a.out_f32) static_cast<float*>(a.C)[o] = acc[mb][nb][r];
        else static_cast<uint16_t*>(a.C)[o] = f32_to_bf16(acc[mb][nb][r]);
      }
    }
  }
}

// Many rows (prefill): LDS-tiled GEMM.  A workgroup of four waves (2 x 2) computes a
// 128 x 256 block of C; each wave a 64 x 128 sub-block, so every operand fragment read
// from LDS feeds 4 or 8 MFMAs (about 96 B/clk of LDS reads per CU at the MFMA rate).
// The A and W tiles of 32 k-columns enter a 3-stage LDS ring by direct global -> LDS
// loads (one KiB per wave instruction: 16 rows of 64 bytes, the 16-byte chunks of a row
// XOR-swizzled by row so that a fragment read hits distinct bank groups); a stage is
// read after its own loads have landed (vmcnt) and a barrier, and the stage two ahead is
// requested right after that barrier.
constexpr int kTBM = 128, kTBN = 256, kTKS = 32, kTStages = 3;
constexpr int kTStageBytes = (kTBM + kTBN) * kTKS * 2;  // 24 KiB

// The 16-byte chunk of a row holding logical chunk c: XOR-swizzled so that 8 (or 16)
// lanes reading one logical chunk of 8 (or 16) consecutive rows hit distinct banks
__device__ __forceinline__ int tile_swz(int row) { return ((row >> 1) & 3) ^ ((row >> 3) & 1); }
__device__ __forceinline__ uint32_t tile_off(int row, int chunk) {
  return static_cast<uint32_t>(row * (kTKS * 2) + ((chunk ^ tile_swz(row)) * 16));
}

__global__ __launch_bounds__(256) void gemm_tiled_kernel(GemmArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[kTStages * kTStageBytes];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int wm = wid >> 1, wn = wid & 1;
  const int64_t batch = blockIdx.z;
  const int64_t bm0 = static_cast<int64_t>(blockIdx.y) * kTBM;
  const int64_t bn0 = static_cast<int64_t>(blockIdx.x) * kTBN;
  const uint16_t* A = a.A + batch * a.sa;
  const uint16_t* W = a.W + batch * a.sw;
  const int nsteps = static_cast<int>(a.K / kTKS);
  const uint32_t lds_b = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds));

  // this wave's 6 of the stage's 24 one-KiB loads: A rows in loads 0..7, W rows in 8..23;
  // lane l of a load fills row 16 i + l / 4 (clamped into the matrix), physical chunk l % 4
  const uint16_t* src[6];
  uint32_t dst[6];
#pragma unroll
  for (int u = 0; u < 6; ++u) {
    const int i = wid + 4 * u;
    const bool isA = i < kTBM / 16;
    const int row = (isA ? i : i - kTBM / 16) * 16 + (lane >> 2);
    const int pc = lane & 3;
    const int c = pc ^ tile_swz(row);
    const int64_t g = isA ? min(bm0 + row, a.M - 1) : min(bn0 + row, a.N - 1);
    src[u] = (isA ? A + g * a.lda : W + g * a.K) + 8 * c;
    dst[u] = static_cast<uint32_t>((isA ? 0 : kTBM * kTKS * 2) + (isA ? i : i - kTBM / 16) * 1024);
  }
  auto issue = [&](int s) {
    const uint32_t base = lds_b + static_cast<uint32_t>((s % kTStages) * kTStageBytes);
#pragma unroll
    for (int u = 0; u < 6; ++u) lds_dma16(src[u] + static_cast<int64_t>(s) * kTKS, base + dst[u]);
  };

  f32x4 acc[4][8];
#pragma unroll
  for (int f = 0; f < 4; ++f)
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) acc[f][nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  if (nsteps > 0) issue(0);
  if (nsteps > 1) issue(1);
  for (int s = 0; s < nsteps; ++s) {
    if (s + 1 < nsteps) wait_vmcnt<6>();
    else wait_vmcnt<0>();
    __syncthreads();  // every wave's part of stage s has landed; stage s - 1 is no longer read
    if (s + 2 < nsteps) issue(s + 2);
    const uint8_t* st = lds + (s % kTStages) * kTStageBytes;
    bf16x8 af[4], wf[8];
#pragma unroll
    for (int f = 0; f < 4; ++f)
      af[f] = *reinterpret_cast<const bf16x8*>(st + tile_off(wm * 64 + 16 * f + col, grp));
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
      wf[nb] = *reinterpret_cast<const bf16x8*>(st + kTBM * kTKS * 2 + tile_off(wn * 128 + 16 * nb + col, grp));
#pragma unroll
    for (int f = 0; f < 4; ++f)
#pragma unroll
      for (int nb = 0; nb < 8; ++nb)
        acc[f][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[f], wf[nb], acc[f][nb], 0, 0, 0);
  }
  // lane (col, grp) holds C[m0 + 4 grp + r][n0 + col] of each 16 x 16 tile
#pragma unroll
  for (int f = 0; f < 4; ++f) {
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) {
      const int64_t n = bn0 + wn * 128 + 16 * nb + col;
      if (n >= a.N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t m = bm0 + wm * 64 + 16 * f + 4 * grp + r;
        if (m >= a.M) continue;
        const int64_t o = batch * a.sc + m * a.ldc + n;
        if (a.out_f32) static_cast<float*>(a.C)[o] = acc[f][nb][r];
        else static_cast<uint16_t*>(a.C)[o] = f32_to_bf16(acc[f][nb][r]);
      }
    }
  }
}

// sums the ksplit partials of every C element in split order
__global__ __launch_bounds__(256) void gemm_reduce_kernel(GemmArgs a) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t per = a.M * a.N;
  if (e >= a.batch * per) return;
  float acc = 0.f;
  for (int s = 0; s < a.ksplit; ++s) acc += a.part[s * a.batch * per + e];
  const int64_t batch = e / per, m = (e % per) / a.N, n = e % a.N;
  const int64_t o = batch * a.sc + m * a.ldc + n;
  if (a.out_f32) static_cast<float*>(a.C)[o] = acc;
  else static_cast<uint16_t*>(a.C)[o] = f32_to_bf16(acc);
}

// the few-rows kernel with the 64-element step
bool few_path(int64_t M, int64_t K) { return M <= kFewRows && K % kFewStep == 0; }

// contraction splits of a GEMM (1 unless few rows leave the chip underfilled)
int gemm_splits(int64_t M, int64_t N, int64_t K, int64_t batch) {
  if (M > kFewRows || M == 0) return 1;
  const int64_t tiles = ((N + 255) / 256) * (few_path(M, K) ? 1 : (M + 15) / 16) * batch;
  const int64_t steps = K / (few_path(M, K) ? kFewStep : kKStep);
  int64_t s = (kTargetGroups + tiles - 1) / tiles;
  s = std::min(s, steps / kMinSplitSteps);
  return static_cast<int>(std::max<int64_t>(s, 1));
}

size_t gemm_part_bytes(int64_t M, int64_t N, int64_t K, int64_t batch) {
  const int s = gemm_splits(M, N, K, batch);
  return s > 1 ? static_cast<size_t>(s) * batch * M * N * sizeof(float) : 0;
}

int launch_gemm(GemmArgs a, int64_t batch, float* part, hipStream_t stream) {
  if (a.M == 0 || a.N == 0 || batch == 0) return 0;
  if (a.K % kKStep) return -2;
  const int steps = static_cast<int>(a.K / (few_path(a.M, a.K) ? kFewStep : kKStep));
  a.batch = batch;
  a.ksplit = gemm_splits(a.M, a.N, a.K, batch);
  a.steps_per_split = (steps + a.ksplit - 1) / a.ksplit;
  a.ksplit = (steps + a.steps_per_split - 1) / a.steps_per_split;  // no empty split
  a.part = part;
  if (a.ksplit > 1 && !part) return -2;
  const uint32_t gz = static_cast<uint32_t>(batch * a.ksplit);
  if (a.M >= kTBM && a.ksplit == 1) {  // many rows: LDS-tiled blocks
    const dim3 g(static_cast<uint32_t>((a.N + kTBN - 1) / kTBN), static_cast<uint32_t>((a.M + kTBM - 1) / kTBM),
                 static_cast<uint32_t>(batch));
    hipLaunchKernelGGL(gemm_tiled_kernel, g, dim3(256), 0, stream, a);
  } else if (few_path(a.M, a.K)) {  // few rows: all rows x 256 columns per workgroup
    const dim3 g(static_cast<uint32_t>((a.N + 255) / 256), 1, gz);
    if (a.M <= 16) hipLaunchKernelGGL((gemm_few_kernel<1>), g, dim3(256), 0, stream, a);
    else hipLaunchKernelGGL((gemm_few_kernel<2>), g, dim3(256), 0, stream, a);
  } else if (a.M <= kFewRows) {  // few rows, contraction not a multiple of 64: 16 x 256 tiles
    const dim3 g(static_cast<uint32_t>((a.N + 255) / 256), static_cast<uint32_t>((a.M + 15) / 16), gz);
    hipLaunchKernelGGL((gemm_bf16_kernel<1, 4>), g, dim3(256), 0, stream, a);
  } else {
    const dim3 g(static_cast<uint32_t>((a.N + 63) / 64), static_cast<uint32_t>((a.M + 63) / 64), gz);
    hipLaunchKernelGGL((gemm_bf16_kernel<4, 1>), g, dim3(256), 0, stream, a);
  }
  if (hipGetLastError() != hipSuccess) return -1;
  if (a.ksplit > 1) {
    const int64_t n = batch * a.M * a.N;
    hipLaunchKernelGGL(gemm_reduce_kernel, dim3(static_cast<uint32_t>((n + 255) / 256)), dim3(256), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return -1;
  }
  return 0;
}

}  // namespace

size_t grouped_out_proj_workspace_bytes(int64_t T, int64_t n_h, int64_t c, int64_t g, int64_t d_g, int64_t d) {
  const size_t mid = (static_cast<size_t>(T) * g * d_g * sizeof(uint16_t) + 255) & ~static_cast<size_t>(255);
  const size_t part = std::max(gemm_part_bytes(T, d_g, (n_h / g) * c, g), gemm_part_bytes(T, d, g * d_g, 1));
  return mid + part;
}

int launch_grouped_out_proj(const GroupedProjLaunch& L, hipStream_t stream) {
  if (L.T == 0) return 0;
  const size_t mid_bytes = (static_cast<size_t>(L.T) * L.g * L.d_g * sizeof(uint16_t) + 255) & ~static_cast<size_t>(255);
  float* part = reinterpret_cast<float*>(static_cast<char*>(L.mid) + mid_bytes);
  const int64_t per = L.n_h / L.g;
  const int64_t K1 = per * L.c;
  GemmArgs a{};
  a.A = static_cast<const uint16_t*>(L.o);
  a.W = static_cast<const uint16_t*>(L.w_group);
  a.C = L.mid;
  a.M = L.T;
  a.N = L.d_g;
  a.K = K1;
  a.lda = L.n_h * L.c;
  a.ldc = L.g * L.d_g;
  a.sa = K1;
  a.sw = L.d_g * K1;
  a.sc = L.d_g;
  a.out_f32 = 0;
  int rc = launch_gemm(a, L.g, part, stream);
  if (rc != 0) return rc;
  GemmArgs b{};
  b.A = static_cast<const uint16_t*>(L.mid);
  b.W = static_cast<const uint16_t*>(L.w_out);
  b.C = L.out;
  b.M = L.T;
  b.N = L.d;
  b.K = L.g * L.d_g;
  b.lda = b.K;
  b.ldc = L.d;
  b.out_f32 = L.out_f32;
  return launch_gemm(b, 1, part, stream);
}

}  // namespace csa
