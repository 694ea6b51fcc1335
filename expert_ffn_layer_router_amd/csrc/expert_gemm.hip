// Grouped expert GEMM: for every expert e, the rows offsets[e] .. offsets[e+1] of A times
// that expert's weight matrix B_e (K x N, row-major "x @ W" layout), with an optional
// epilogue: ReLU (the two-layer ReLU expert's hidden layer, Sparsely-Gated Layer page,
// expert_forward) or SwiGLU silu(A B0_e) * (A B1_e) (the SwiGLU expert named on the ML
// Grind page, Background). Each expert runs only on its own rows (ML Grind, Constraints).
//
// The tile schedule is read from the device-side offsets: the grid (x: M-tiles, y: N-tiles)
// is sized for the worst case (sum over experts of ceil(rows_e / BM) <= ceil(max_rows / BM) + E M-tiles), and
// each block maps its M-tile id to (expert, first row) with a wave-wide prefix sum over
// the per-expert tile counts; blocks past the last tile exit at once.
//
// bf16 path: v_mfma_f32_32x32x16_bf16 (gfx950), fp32 accumulation, LDS-staged tiles.
// The weights are N-contiguous, while the MFMA operand wants 8 consecutive K values per
// lane, so the B tile is transposed on its way into LDS (4 K-rows x 8 columns per thread,
// repacked in registers). Optional row gather: row r of A is A[a_gather[r] / gather_div],
// which lets the layer feed token rows straight from x without a permuted copy.
#include "common.hpp"
#include "tile_schedule.hpp"

namespace moe {
namespace {

__device__ __forceinline__ uint32_t lo16(uint32_t w) { return w & 0xffffu; }
__device__ __forceinline__ uint32_t hi16(uint32_t w) { return w >> 16; }

constexpr int kBM = 128, kBN = 128, kBK = 64;
constexpr int kLds = kBK + 8;  // padded row stride (elements) of the LDS tiles
constexpr int kThreads = 256;

// Global -> registers: the A tile (4 rows of 8 K-values per thread) and the B tile(s)
// (4 K-rows of 8 columns per thread).
template <int NB>
__device__ __forceinline__ void load_tiles(uint4 (&ra)[4], uint4 (&rb)[NB][4],
                                           const uint16_t* const (&a_src)[4],
                                           const uint16_t* const (&Bm)[NB], int64_t k0, int64_t K,
                                           int64_t N, int a_kc, int b_kq, bool b_ok,
                                           int64_t b_col) {
  const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int64_t kk = k0 + a_kc;
    ra[p] = zero;
    if (a_src[p] && kk < K) ra[p] = *(const uint4*)(a_src[p] + kk);
  }
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t kr = k0 + 4 * b_kq + i;
      rb[nb][i] = zero;
      if (b_ok && kr < K) rb[nb][i] = *(const uint4*)(Bm[nb] + kr * N + b_col);
    }
}

// Registers -> LDS. A keeps its layout; each 4 x 8 block of B is transposed so that LDS
// holds, for every column, its K values contiguously (the MFMA operand layout).
template <int NB>
__device__ __forceinline__ void store_tiles(const uint4 (&ra)[4], const uint4 (&rb)[NB][4],
                                            uint16_t* sA, uint16_t (*sB)[kBN * kLds], int tid,
                                            int a_kc, int b_kq, int b_nb) {
#pragma unroll
  for (int p = 0; p < 4; ++p) *(uint4*)&sA[((tid >> 3) + 32 * p) * kLds + a_kc] = ra[p];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) {
    const uint32_t w0[4] = {rb[nb][0].x, rb[nb][0].y, rb[nb][0].z, rb[nb][0].w};
    const uint32_t w1[4] = {rb[nb][1].x, rb[nb][1].y, rb[nb][1].z, rb[nb][1].w};
    const uint32_t w2[4] = {rb[nb][2].x, rb[nb][2].y, rb[nb][2].z, rb[nb][2].w};
    const uint32_t w3[4] = {rb[nb][3].x, rb[nb][3].y, rb[nb][3].z, rb[nb][3].w};
#pragma unroll
    for (int wi = 0; wi < 4; ++wi) {
      // columns 2wi (low halves) and 2wi+1 (high halves)
      const uint32_t lo01 = lo16(w0[wi]) | (lo16(w1[wi]) << 16);
      const uint32_t lo23 = lo16(w2[wi]) | (lo16(w3[wi]) << 16);
      const uint32_t hi01 = hi16(w0[wi]) | (hi16(w1[wi]) << 16);
      const uint32_t hi23 = hi16(w2[wi]) | (hi16(w3[wi]) << 16);
      *(uint2*)&sB[nb][(8 * b_nb + 2 * wi) * kLds + 4 * b_kq] = make_uint2(lo01, lo23);
      *(uint2*)&sB[nb][(8 * b_nb + 2 * wi + 1) * kLds + 4 * b_kq] = make_uint2(hi01, hi23);
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(kThreads, 2) void gemm_bf16_mfma_kernel(const GroupedGemm g) {
  constexpr int NB = (EPI == EPI_SWIGLU) ? 2 : 1;
  __shared__ __align__(16) uint16_t sA[kBM * kLds];
  __shared__ __align__(16) uint16_t sB[NB][kBN * kLds];

  int e, row0, rows;
  if (!find_tile(g.offsets, g.E, kBM, (int)blockIdx.x, e, row0, rows)) return;
  const int64_t K = g.K, N = g.N;
  const int64_t n0 = (int64_t)blockIdx.y * kBN;
  const int tid = threadIdx.x, lane = lane_id(), wv = wave_id();
  const int wm = wv >> 1, wn = wv & 1;  // 2 x 2 waves, 64 x 64 each

  // A loads: rows tid/8 + 32p (p < 4), 8 K-values at (tid % 8) * 8.
  const uint16_t* A = (const uint16_t*)g.A;
  const uint16_t* a_src[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int r = (tid >> 3) + 32 * p;
    a_src[p] = nullptr;
    if (r < rows) {
      const int64_t gr = row0 + r;
      const int64_t src = g.a_gather ? (int64_t)(g.a_gather[gr] / g.gather_div) : gr;
      a_src[p] = A + src * g.lda;
    }
  }
  const int a_kc = (tid & 7) * 8;

  // B loads: K rows 4*(tid/16) .. +3, columns 8*(tid%16) .. +7.
  const int b_kq = tid >> 4, b_nb = tid & 15;
  const int64_t b_col = n0 + 8 * b_nb;
  const bool b_ok = b_col < N;  // N % 8 == 0: a vector is all in or all out
  const uint16_t* Bm[NB];
  Bm[0] = (const uint16_t*)g.B0 + (int64_t)e * K * N;
  if (NB == 2) Bm[NB - 1] = (const uint16_t*)g.B1 + (int64_t)e * K * N;

  uint4 ra[4], rb[NB][4];
  f32x16 acc[NB][2][2];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
      for (int ni = 0; ni < 2; ++ni)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[nb][mi][ni][v] = 0.f;

  load_tiles<NB>(ra, rb, a_src, Bm, 0, K, N, a_kc, b_kq, b_ok, b_col);
  for (int64_t k0 = 0; k0 < K; k0 += kBK) {
    __syncthreads();
    store_tiles<NB>(ra, rb, sA, sB, tid, a_kc, b_kq, b_nb);
    __syncthreads();
    if (k0 + kBK < K) load_tiles<NB>(ra, rb, a_src, Bm, k0 + kBK, K, N, a_kc, b_kq, b_ok, b_col);
#pragma unroll
    for (int kk = 0; kk < kBK; kk += 16) {
      bf16x8 a[2], b[NB][2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
        a[mi] = *(const bf16x8*)&sA[(wm * 64 + mi * 32 + (lane & 31)) * kLds + kk + (lane >> 5) * 8];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          b[nb][ni] =
              *(const bf16x8*)&sB[nb][(wn * 64 + ni * 32 + (lane & 31)) * kLds + kk + (lane >> 5) * 8];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int mi = 0; mi < 2; ++mi)
#pragma unroll
          for (int ni = 0; ni < 2; ++ni)
            acc[nb][mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], b[nb][ni],
                                                                      acc[nb][mi][ni], 0, 0, 0);
    }
  }

  // 32x32 accumulator layout: lane l holds column l % 32, rows 8*(v/4) + 4*(l/32) + v%4.
  uint16_t* C = (uint16_t*)g.C;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int r = wm * 64 + mi * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        const int64_t col = n0 + wn * 64 + ni * 32 + (lane & 31);
        if (r < rows && col < N) {
          float val = acc[0][mi][ni][v];
          if (EPI == EPI_RELU) val = fmaxf(val, 0.f);
          if (EPI == EPI_SWIGLU) {
            const float up = acc[NB - 1][mi][ni][v];
            val = val / (1.f + __expf(-val)) * up;
          }
          C[(int64_t)(row0 + r) * N + col] = f32_to_bf16(val);
        }
      }
}

// float32 path (VALU, 64 x 64 tiles, 4 x 4 outputs per thread). Any K and N.
constexpr int kFBM = 64, kFBN = 64, kFBK = 16;

template <int EPI>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(const GroupedGemm g) {
  constexpr int NB = (EPI == EPI_SWIGLU) ? 2 : 1;
  __shared__ float sA[kFBK][kFBM + 4];
  __shared__ float sB[NB][kFBK][kFBN + 4];
  int e, row0, rows;
  if (!find_tile(g.offsets, g.E, kFBM, (int)blockIdx.x, e, row0, rows)) return;
  const int64_t K = g.K, N = g.N;
  const int64_t n0 = (int64_t)blockIdx.y * kFBN;
  const int tid = threadIdx.x, ty = tid >> 4, tx = tid & 15;
  const float* A = (const float*)g.A;
  const float* Bm[NB];
  Bm[0] = (const float*)g.B0 + (int64_t)e * K * N;
  if (NB == 2) Bm[NB - 1] = (const float*)g.B1 + (int64_t)e * K * N;

  float acc[NB][4][4];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[nb][i][j] = 0.f;

  for (int64_t k0 = 0; k0 < K; k0 += kFBK) {
    for (int i = tid; i < kFBM * kFBK; i += kThreads) {
      const int r = i / kFBK, kk = i % kFBK;
      float v = 0.f;
      if (r < rows && k0 + kk < K) {
        const int64_t gr = row0 + r;
        const int64_t src = g.a_gather ? (int64_t)(g.a_gather[gr] / g.gather_div) : gr;
        v = A[src * g.lda + k0 + kk];
      }
      sA[kk][r] = v;
    }
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
      for (int i = tid; i < kFBK * kFBN; i += kThreads) {
        const int kk = i / kFBN, c = i % kFBN;
        sB[nb][kk][c] = (k0 + kk < K && n0 + c < N) ? Bm[nb][(k0 + kk) * N + n0 + c] : 0.f;
      }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < kFBK; ++kk) {
      float a[4], b[NB][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = sA[kk][ty * 4 + i];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int j = 0; j < 4; ++j) b[nb][j] = sB[nb][kk][tx * 4 + j];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[nb][i][j] = fmaf(a[i], b[nb][j], acc[nb][i][j]);
    }
    __syncthreads();
  }
  float* C = (float*)g.C;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int r = ty * 4 + i;
      const int64_t col = n0 + tx * 4 + j;
      if (r < rows && col < N) {
        float val = acc[0][i][j];
        if (EPI == EPI_RELU) val = fmaxf(val, 0.f);
        if (EPI == EPI_SWIGLU) val = val / (1.f + expf(-val)) * acc[NB - 1][i][j];
        C[(int64_t)(row0 + r) * N + col] = val;
      }
    }
}

}  // namespace

hipError_t launch_grouped_gemm(const GroupedGemm& g, hipStream_t s) {
  if (g.max_rows <= 0 || g.N <= 0) return hipSuccess;
  // the 256 x 256 kernel needs K % 128 == 0; other bf16 shapes take the 128 x 128 kernel
  if (g.k_grouped)  // only the 256 x 256 kernel has this mode
    return (g.dtype == MOE_BF16 && g.queue && g.epilogue == EPI_NONE && !g.b_kmajor)
               ? launch_grouped_gemm_bf16_256(g, s)
               : hipErrorInvalidValue;
  const bool k256 = g.dtype == MOE_BF16 && g.K % 128 == 0 && g.queue;
  if (g.b_kmajor && (!k256 || g.epilogue != EPI_NONE)) return hipErrorInvalidValue;
  if ((g.pre_a || g.pre_b) &&
      (!k256 || g.epilogue == EPI_NONE || !g.pre_a || (g.epilogue == EPI_SWIGLU) != (g.pre_b != nullptr)))
    return hipErrorInvalidValue;
  if (k256) return launch_grouped_gemm_bf16_256(g, s);
  if (g.ev_start) hipEventRecord(g.ev_start, s);
  if (g.dtype == MOE_BF16) {
    const int64_t mt = (g.max_rows + kBM - 1) / kBM + g.E;
    const dim3 grid((unsigned)mt, (unsigned)((g.N + kBN - 1) / kBN));
    switch (g.epilogue) {
      case EPI_NONE:
        hipLaunchKernelGGL(gemm_bf16_mfma_kernel<EPI_NONE>, grid, dim3(kThreads), 0, s, g);
        break;
      case EPI_RELU:
        hipLaunchKernelGGL(gemm_bf16_mfma_kernel<EPI_RELU>, grid, dim3(kThreads), 0, s, g);
        break;
      default:
        hipLaunchKernelGGL(gemm_bf16_mfma_kernel<EPI_SWIGLU>, grid, dim3(kThreads), 0, s, g);
        break;
    }
  } else {
    const int64_t mt = (g.max_rows + kFBM - 1) / kFBM + g.E;
    const dim3 grid((unsigned)mt, (unsigned)((g.N + kFBN - 1) / kFBN));
    switch (g.epilogue) {
      case EPI_NONE:
        hipLaunchKernelGGL(gemm_f32_kernel<EPI_NONE>, grid, dim3(kThreads), 0, s, g);
        break;
      case EPI_RELU:
        hipLaunchKernelGGL(gemm_f32_kernel<EPI_RELU>, grid, dim3(kThreads), 0, s, g);
        break;
      default:
        hipLaunchKernelGGL(gemm_f32_kernel<EPI_SWIGLU>, grid, dim3(kThreads), 0, s, g);
        break;
    }
  }
  if (g.ev_stop) hipEventRecord(g.ev_stop, s);
  return hipGetLastError();
}

}  // namespace moe
