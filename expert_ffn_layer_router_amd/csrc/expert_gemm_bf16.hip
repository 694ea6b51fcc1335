// Grouped expert GEMM, bf16 storage / fp32 accumulation, for gfx950 (the expert FFN of the
// layer: each expert runs only on its own rows, ML Grind "Mixture-of-Experts (MoE) Routing",
// Constraints; SwiGLU and ReLU experts as on the ML Grind and Sparsely-Gated Layer pages).
//
// Tiling (one 256-thread block per 256 x 256 output tile, one block per CU):
//  * 4 waves stacked along M; wave w owns rows 64w .. 64w+63 of the tile and all 256
//    columns, i.e. 4 x 16 MFMA tiles of 16x16 (v_mfma_f32_16x16x32_bf16) and 256 fp32
//    accumulators per lane.
//  * A (activations, K-contiguous rows) goes straight from global memory into the MFMA
//    operand registers: lane l of m-tile i loads row 16i + l%16, K values 8(l/16)..+7, which
//    is exactly the operand layout. No LDS, and a row gather (token rows of x through the
//    dispatch permutation) costs nothing extra.
//  * B (expert weights, (K, N) row-major, N-contiguous) is shared by the 4 waves through LDS.
//    Each thread loads an 8 (K) x 8 (N) block with eight 16-byte loads, transposes it in
//    registers and writes eight 16-byte K-runs, so every wave then reads its MFMA B operands
//    with conflict-free ds_read_b128 (row stride 144 bytes).
//  * BK = 64 per stage (K % 128 == 0 is required); A is double-buffered in registers and B
//    in LDS, so the global loads of stage s+1 are in flight while stage s computes. Loads
//    are never masked: rows and columns past the tile read valid memory whose results are
//    never stored.
//  * SwiGLU: the 256 columns interleave 16-column tiles of W1 and W3 for the same 128
//    output columns, so each lane holds the gate and the up value of the same output and the
//    epilogue silu(gate) * up needs no data exchange.
//  * Tile order: expert by expert, in blocks of (that expert's M-tiles) x 8 column tiles with
//    the M-tiles fastest; blockIdx is remapped so each XCD (blocks b with the same b % 8)
//    works through a contiguous range of that order. The ~32 tiles an XCD runs at once then
//    share a few activation row blocks and a few weight column blocks in its own L2.
#include "common.hpp"
#include "tile_schedule.hpp"

namespace moe {
namespace {

constexpr int kBM = 256, kBK = 64;
constexpr int kLds = kBK + 8;  // elements per LDS column (144 bytes)
constexpr int kThreads = 256;
constexpr int kTileBlockN = 8;  // column tiles per L2-sharing block of one expert

__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return (a & 0xffffu) | (b << 16);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return (a >> 16) | (b & 0xffff0000u);
}

// Global loads as a block-uniform base plus a 32-bit per-lane byte offset, so each load is
// one instruction with the base in scalar registers (no 64-bit address per lane and load).
__device__ __forceinline__ uint4 gload(const char* base, uint32_t off) {
  return *(const uint4*)(base + off);
}

__device__ __forceinline__ uint4 select4(bool keep, const uint4& v) {
  return make_uint4(keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u);
}

struct BLoader {
  const char* base;  // this expert's weight matrix (block-uniform)
  uint32_t col_off;  // byte offset of this thread's 8-column block (column 0 if past N)
  uint32_t row_bytes;
  int kq;            // 8-row group of K within a stage
  int64_t K;
};

// 8 rows (K) x 8 columns (N) of the weight tile for stage k0 (this kernel requires
// K % 64 == 0). Columns past N read column 0 of the block instead (valid memory; those
// outputs are never stored), so no load is masked or branched around.
__device__ __forceinline__ void load_b(const BLoader& bl, int64_t k0, uint4 (&rb)[8]) {
  const uint32_t o0 = bl.col_off + (uint32_t)(k0 + 8 * bl.kq) * bl.row_bytes;
#pragma unroll
  for (int i = 0; i < 8; ++i) rb[i] = gload(bl.base, o0 + i * bl.row_bytes);
}

// Transposed into LDS: column c of the block gets its 8 K values as one 16-byte run.
__device__ __forceinline__ void store_b(uint16_t* sb, int cb, int kq, const uint4 (&rb)[8]) {
  uint32_t w[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    w[i][0] = rb[i].x;
    w[i][1] = rb[i].y;
    w[i][2] = rb[i].z;
    w[i][3] = rb[i].w;
  }
#pragma unroll
  for (int d = 0; d < 4; ++d) {
    // columns 2d (low halves) and 2d+1 (high halves)
    const uint4 lo = make_uint4(pack_lo(w[0][d], w[1][d]), pack_lo(w[2][d], w[3][d]),
                                pack_lo(w[4][d], w[5][d]), pack_lo(w[6][d], w[7][d]));
    const uint4 hi = make_uint4(pack_hi(w[0][d], w[1][d]), pack_hi(w[2][d], w[3][d]),
                                pack_hi(w[4][d], w[5][d]), pack_hi(w[6][d], w[7][d]));
    *(uint4*)&sb[(8 * cb + 2 * d) * kLds + 8 * kq] = lo;
    *(uint4*)&sb[(8 * cb + 2 * d + 1) * kLds + 8 * kq] = hi;
  }
}

// A operands of one stage: 2 m-tiles of 32 rows x 4 k-steps of 16. Rows past the tile read
// row 0 of A (valid memory; their outputs are never stored).
__device__ __forceinline__ void load_a(const char* abase, const uint32_t (&aoff)[2], int64_t k0,
                                       uint4 (&ra)[2][4]) {
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int t = 0; t < 4; ++t) ra[mi][t] = gload(abase, aoff[mi] + (uint32_t)(k0 + 16 * t) * 2u);
}

__device__ __forceinline__ bf16x8 read_b(const uint16_t* sb, int c, int t, int lane) {
  return *(const bf16x8*)&sb[(32 * c + (lane & 31)) * kLds + 16 * t + 8 * (lane >> 5)];
}

template <int NTW>
__device__ __forceinline__ void read_bs(const uint16_t* sb, int t, int lane, bf16x8 (&b)[NTW]) {
#pragma unroll
  for (int c = 0; c < NTW; ++c) b[c] = read_b(sb, c, t, lane);
}

template <int NTW>
__device__ __forceinline__ void mfma_step(const uint4 (&ra)[2][4], int t, const bf16x8 (&b)[NTW],
                                          f32x16 (&acc)[2][NTW]) {
  const bf16x8 a0 = __builtin_bit_cast(bf16x8, ra[0][t]);
  const bf16x8 a1 = __builtin_bit_cast(bf16x8, ra[1][t]);
#pragma unroll
  for (int c = 0; c < NTW; ++c) {
    acc[0][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b[c], acc[0][c], 0, 0, 0);
    acc[1][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b[c], acc[1][c], 0, 0, 0);
  }
}

// 4 k-steps of 16, each 2 row tiles x NTW column tiles of v_mfma_f32_32x32x16_bf16. The B
// operands of k-step t+1 are read from LDS while the MFMAs of k-step t run; scheduling
// fences keep the compiler from sinking those reads next to their uses.
template <int NTW>
__device__ __forceinline__ void compute_stage(const uint16_t* sb, const uint4 (&ra)[2][4],
                                              int lane, f32x16 (&acc)[2][NTW]) {
  bf16x8 b0[NTW], b1[NTW];
  read_bs<NTW>(sb, 0, lane, b0);
  __builtin_amdgcn_sched_barrier(0);
  read_bs<NTW>(sb, 1, lane, b1);
  __builtin_amdgcn_sched_barrier(0);
  mfma_step<NTW>(ra, 0, b0, acc);
  __builtin_amdgcn_sched_barrier(0);
  read_bs<NTW>(sb, 2, lane, b0);
  __builtin_amdgcn_sched_barrier(0);
  mfma_step<NTW>(ra, 1, b1, acc);
  __builtin_amdgcn_sched_barrier(0);
  read_bs<NTW>(sb, 3, lane, b1);
  __builtin_amdgcn_sched_barrier(0);
  mfma_step<NTW>(ra, 2, b0, acc);
  __builtin_amdgcn_sched_barrier(0);
  mfma_step<NTW>(ra, 3, b1, acc);
}

// NTW = column tiles of 32 per wave: 8 gives 256 x 256 tiles at one block per CU, 4 gives
// 256 x 128 tiles with two blocks per CU (each wave hides the other's LDS latency).
template <int EPI, int NTW>
__global__ __launch_bounds__(kThreads, 8 / NTW) void gemm_bf16_256_kernel(const GroupedGemm g,
                                                                          int nt) {
  constexpr bool kSwiGLU = EPI == EPI_SWIGLU;
  constexpr int kBN = 32 * NTW;
  __shared__ __align__(16) uint16_t sB[2][kBN * kLds];

  // XCD-aware order: XCD x (= blockIdx % 8) takes the x-th contiguous eighth of the tiles.
  const int b = blockIdx.x;
  int e, row0, rows, n_tile;
  if (!find_tile_2d(g.offsets, g.E, kBM, nt, kTileBlockN, b, e, row0, rows, n_tile)) return;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t K = g.K, N = g.N;
  const int64_t n0 = (int64_t)n_tile * (kSwiGLU ? kBN / 2 : kBN);  // first output column
  if (n0 >= N) return;

  // A: this lane's 4 rows (one per m-tile) and its K offset inside each 32-step
  const char* abase = (const char*)g.A;
  const int koff = 8 * (lane >> 5);
  uint32_t aoff[2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
    const int r = 64 * wv + 32 * mi + (lane & 31);
    int64_t src = 0;
    if (r < rows) {
      const int64_t gr = row0 + r;
      src = g.a_gather ? (int64_t)(g.a_gather[gr] / g.gather_div) : gr;
    }
    aoff[mi] = (uint32_t)((src * g.lda + koff) * 2);
  }

  // B: thread -> (8-column block cb of the tile columns, 8-row group kq of the stage). With
  // 128-column tiles the upper 128 threads load a copy of the lower half's blocks (so every
  // thread issues the same loads and the wait counts stay static) and do not store them.
  const int cb = tid >> 3, kq = tid & 7;
  const bool b_loader = cb < kBN / 8;
  BLoader bl;
  {
    int64_t col;
    const uint16_t* Wm;
    const int cbl = cb % (kBN / 8);
    if (kSwiGLU) {
      const int c = cbl >> 2;  // tile column block of 32: even -> W1, odd -> W3
      Wm = (const uint16_t*)((c & 1) ? g.B1 : g.B0);
      col = n0 + 32 * (c >> 1) + 8 * (cbl & 3);
    } else {
      Wm = (const uint16_t*)g.B0;
      col = n0 + 8 * cbl;
    }
    bl.base = (const char*)(Wm + (int64_t)e * K * N);
    bl.col_off = (uint32_t)((col < N ? col : 0) * 2);
    bl.row_bytes = (uint32_t)(N * 2);
    bl.K = K;
    bl.kq = kq;
  }

  f32x16 acc[2][NTW];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int c = 0; c < NTW; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[mi][c][v] = 0.f;

  const bool active = 64 * wv < rows;  // this wave has rows to store
  const int nst = (int)(K / kBK);       // even: K % (2 * kBK) == 0 is required
  uint4 ra0[2][4], ra1[2][4], rb[8];

  load_a(abase, aoff, 0, ra0);
  load_b(bl, 0, rb);
  if (b_loader) store_b(sB[0], cb, kq, rb);
  __syncthreads();

  // Stage s computes from registers ra(s%2) and LDS buffer s%2 while the loads of stage s+1
  // are in flight; B of stage s+1 then goes to the other LDS buffer. Every iteration is the
  // same (no tail, no conditional loads), so each wait covers exactly the operands it needs;
  // the prefetch past the last stage re-reads the last stage (valid memory) and is unused.
  // Every wave computes, including waves whose rows are all past the tile (their results are
  // not stored): a branch around the MFMAs would make the compiler copy accumulators.
  for (int s = 0; s < nst; s += 2) {
    const int64_t k1 = (int64_t)(s + 1) * kBK;
    const int64_t k2 = (int64_t)min(s + 2, nst - 1) * kBK;
    load_a(abase, aoff, k1, ra1);
    load_b(bl, k1, rb);
    compute_stage<NTW>(sB[0], ra0, lane, acc);
    if (b_loader) store_b(sB[1], cb, kq, rb);
    __syncthreads();
    load_a(abase, aoff, k2, ra0);
    load_b(bl, k2, rb);
    compute_stage<NTW>(sB[1], ra1, lane, acc);
    if (b_loader) store_b(sB[0], cb, kq, rb);
    __syncthreads();
  }

  if (!active) return;
  // 32x32 accumulator layout: lane l holds column l % 32, rows 8*(v/4) + 4*(l/32) + v%4.
  uint16_t* C = (uint16_t*)g.C;
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int r = 64 * wv + 32 * mi + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
      if (r >= rows) continue;
      uint16_t* crow = C + (int64_t)(row0 + r) * N;
      if (kSwiGLU) {
#pragma unroll
        for (int q = 0; q < NTW / 2; ++q) {
          const int64_t col = n0 + 32 * q + (lane & 31);
          if (col < N) {
            const float gt = acc[mi][2 * q][v], up = acc[mi][2 * q + 1][v];
            crow[col] = f32_to_bf16(gt / (1.f + __expf(-gt)) * up);
          }
        }
      } else {
#pragma unroll
        for (int c = 0; c < NTW; ++c) {
          const int64_t col = n0 + 32 * c + (lane & 31);
          if (col < N) {
            float val = acc[mi][c][v];
            if (EPI == EPI_RELU) val = fmaxf(val, 0.f);
            crow[col] = f32_to_bf16(val);
          }
        }
      }
    }
}

template <int NTW>
hipError_t launch_ntw(const GroupedGemm& g, hipStream_t s) {
  constexpr int kBN = 32 * NTW;
  const int64_t mt_max = (g.max_rows + kBM - 1) / kBM + g.E;
  const int64_t cols = (g.epilogue == EPI_SWIGLU) ? kBN / 2 : kBN;
  const int64_t nt = (g.N + cols - 1) / cols;
  int64_t G = mt_max * nt;
  G = (G + 7) / 8 * 8;
  const dim3 grid((unsigned)G);
  switch (g.epilogue) {
    case EPI_NONE:
      hipLaunchKernelGGL((gemm_bf16_256_kernel<EPI_NONE, NTW>), grid, dim3(kThreads), 0, s, g,
                         (int)nt);
      break;
    case EPI_RELU:
      hipLaunchKernelGGL((gemm_bf16_256_kernel<EPI_RELU, NTW>), grid, dim3(kThreads), 0, s, g,
                         (int)nt);
      break;
    default:
      hipLaunchKernelGGL((gemm_bf16_256_kernel<EPI_SWIGLU, NTW>), grid, dim3(kThreads), 0, s, g,
                         (int)nt);
      break;
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_gemm_bf16_256(const GroupedGemm& g, hipStream_t s) {
  return launch_ntw<8>(g, s);
}

}  // namespace moe
