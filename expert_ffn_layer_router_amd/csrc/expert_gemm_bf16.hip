// Grouped expert GEMM, bf16 storage / fp32 accumulation, for gfx950 (the expert FFN of the
// layer: each expert runs only on its own rows, ML Grind "Mixture-of-Experts (MoE) Routing",
// Constraints; SwiGLU and ReLU experts as on the ML Grind and Sparsely-Gated Layer pages).
//
// One 256-thread block per 256 x 256 output tile, one block per CU; 4 waves stacked along M,
// wave w owning rows 64w .. 64w+63 and all 256 columns (2 x 8 tiles of
// v_mfma_f32_32x32x16_bf16, 256 fp32 accumulators per lane).
//
// Both operands go from global memory straight into LDS with global_load_lds_dwordx4 (lane l
// of an instruction writes 16 bytes at the instruction's LDS base + 16 l). A stage is 32 of K:
//  * A (activations, 256 rows x 32 K, 64 bytes a row): an instruction fills 16 rows; 16-byte
//    chunk c of row r is stored at chunk c ^ ((r / 4) % 4), which makes the MFMA operand
//    reads (ds_read_b128: 16 rows x 16 bytes per 16 lanes, 64 banks) conflict-free. A row
//    gather (token rows of x through the dispatch permutation) is just a per-lane source
//    address.
//  * B (weights, 32 K-rows x 256 columns, (K, N) row-major, 512 bytes a row): an instruction
//    fills 2 K-rows; chunk c of K-row k is stored at c ^ (4 (k % 4)), and the MFMA operands
//    come from transposed reads (ds_read_b64_tr_b16), which turn the N-contiguous layout into
//    8 consecutive K values per lane.
// Four stage buffers (A then B, 32 KB each, 128 KB in all), used in rotation: every unit (a
// tile, or a K part of one) has a multiple of four stages, so stage s of any unit uses buffer
// s % 4 and the stage loop is written out four stages a trip, with every LDS offset a
// constant. The loads of a stage are issued four stages before it is computed, so about three stages (96 KB per CU)
// are in flight while the waves compute. The block synchronises once per stage, before the
// stage's last k-step: that k-step's operands are already in registers, so its MFMAs cover
// the reads of the next buffer's first operands and the issue of the loads four stages ahead
// into the buffer just finished. The loads are issued from inline assembly, so the compiler
// does not track them; every wait for them is explicit and counted: before the barrier that
// publishes stage s + 1, a wave lets only its loads of the two stages after it stay in
// flight (s_waitcnt vmcnt(16), 8 loads per wave and stage; vector memory operations
// complete in issue order).
//  * SwiGLU: the 256 columns interleave 32-column tiles of W1 and W3 for the same 128 output
//    columns, so each lane holds the gate and the up value of the same output.
//  * Epilogue: lanes l and l ^ 1 hold adjacent columns; one swap per pair of rows lets each
//    lane convert two outputs with one v_cvt_pk_bf16_f32 and store them in 4 bytes.
//  * Tile order: expert by expert, in blocks of (that expert's M-tiles) x 8 column tiles with
//    the M-tiles fastest (when the launch's split-K tail can hold every expert's short last
//    tile, those go last and make up the tail); each XCD (blocks b with the same b % 8) works
//    through a contiguous eighth of the real tiles, so the tiles it runs at once share rows and
//    columns in its L2.
#include <hip/hip_ext.h>

#include <type_traits>

#include <limits.h>

#include "common.hpp"
#include "tile_schedule.hpp"

namespace moe {
namespace {

constexpr int kBM = 256, kBN = 256, kBK = 32;
constexpr int kThreads = 256;
constexpr int kTileBlockM = 4;       // M-tiles per L2-sharing block of one group (wgrad)
constexpr int kTileBlockN = 8;       // column tiles per L2-sharing block of one expert
constexpr int kNBuf = 4;             // stage buffers; loads run kNBuf stages ahead
constexpr uint32_t kHalf = kBK * 256 * 2;  // bytes of one stage of either operand (16 KB)
constexpr uint32_t kBuf = 2 * kHalf;       // one stage buffer: A then B (32 KB)
constexpr int kKeep = (kNBuf - 2) * 8;     // own loads a stage wait leaves in flight
constexpr int kMaxSplit = 4;         // K parts of a tail tile at most
constexpr int kMinPartStages = 64;   // K stages of a part at least (K >= 2048 per part)

typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4i16;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt bits 3:0 and 15:14)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4));
}
// The same for a wave-uniform keep of 0, 8, 16, 24 or 32 loads (a scalar branch to the
// matching immediate; any other value waits for everything).
__device__ __forceinline__ void wait_keep(int keep) {
  switch (keep) {
    case 8: wait_vm_lgkm0<8>(); break;
    case 16: wait_vm_lgkm0<16>(); break;
    case 24: wait_vm_lgkm0<24>(); break;
    case 32: wait_vm_lgkm0<32>(); break;
    default: wait_vm_lgkm0<0>(); break;
  }
}
__device__ __forceinline__ void block_barrier() { asm volatile("s_barrier" ::: "memory"); }

struct Loader {
  const char* a[4];  // A source of this lane for instruction j, at K = 0
  const char* bt[4]; // K-major B (the transposed-weight mode): like a[], rows are columns
  const char* b[2];  // B source of this lane for instructions with j % 2 == q, at K-row 0
  int64_t b_row_bytes;
};

// One global_load_lds_dwordx4: 16 bytes per lane from p + off to LDS byte address
// lds + 16 * lane (off and lds are wave-uniform, off held in SGPRs). No register receives
// data, so nothing in the wave depends on it until an explicit s_waitcnt vmcnt. The 64-bit add
// is written next to the load, so that a stage's address arithmetic is one VALU operation per
// load (left to itself the compiler rebuilt the addresses with 64-bit multiply-adds in every
// stage, between the MFMAs).
__device__ __forceinline__ void dma16_at(const void* p, int64_t off, uint32_t lds) {
  uint64_t t;
  asm volatile("v_lshl_add_u64 %0, %1, 0, %2\n\ts_mov_b32 m0, %3\n\ts_nop 0\n\t"
               "global_load_lds_dwordx4 %0, off"
               : "=&v"(t)
               : "v"(p), "s"(off), "s"(lds)
               : "memory", "m0");
}

// Load d (0..7) of this wave for a stage at K offset k0 into the buffer at LDS byte address
// sa: even d -> A instruction d / 2 (16 rows), odd d -> B instruction d / 2 (2 K-rows). bk is
// k0 times B's row pitch in bytes. With BT (B stored K-major, (N, K) per expert), B's stage is
// laid out and loaded exactly like A's: 256 columns x 32 K, 64 bytes a column, an instruction
// fills 16 columns.
template <bool BT>
__device__ __forceinline__ void load_one(const Loader& ld, int64_t k0, int64_t bk, uint32_t sa,
                                         int wv, int d) {
  const int j = d >> 1;
  if (d & 1) {
    if (BT)
      dma16_at(ld.bt[j], k0 * 2, sa + kHalf + (4 * wv + j) * 1024);
    else
      dma16_at(ld.b[j & 1], bk + (int64_t)(2 * j) * ld.b_row_bytes,
               sa + kHalf + (4 * wv + j) * 1024);
  } else {
    dma16_at(ld.a[j], k0 * 2, sa + (4 * wv + j) * 1024);
  }
}
template <bool BT>
__device__ __forceinline__ void load_stage(const Loader& ld, int64_t k0, uint32_t sa, int wv) {
  const int64_t bk = k0 * ld.b_row_bytes;
#pragma unroll
  for (int d = 0; d < 8; ++d) load_one<BT>(ld, k0, bk, sa, wv, d);
}

typedef __attribute__((address_space(3))) const char lds_cchar;

// B operand of n-tile c, k-step t: two transposed 8-byte reads (K-rows 16t + 8 (lane/32) + 4h
// + (lane%16)/4, see the offsets in the kernel) give column lane % 32, K values
// 16t + 8 (lane / 32) .. +7.
__device__ __forceinline__ bf16x8 read_b(const uint32_t (&bb)[4], int c, int t) {
  lds_cchar* p = (lds_cchar*)(uintptr_t)bb[c & 3] + (c & 4) * 64 + t * 16 * 512;
  const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)p);
  const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4i16*)(p + 4 * 512));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// K-major B operand (BT) of column tile c, k-step t: read like A, from bases bb[t].
__device__ __forceinline__ bf16x8 read_bt(const uint32_t (&bb)[4], int c, int t) {
  return *(const lds_bf16x8*)((lds_cchar*)(uintptr_t)bb[t] + c * 32 * 64);
}
template <bool BT>
__device__ __forceinline__ bf16x8 read_b_any(const uint32_t (&bb)[4], int c, int t) {
  return BT ? read_bt(bb, c, t) : read_b(bb, c, t);
}

// A operand of m-tile mi, k-step t: row 64 w + 32 mi + lane % 32, K values 16t + 8 (lane/32)..
__device__ __forceinline__ bf16x8 read_a(const uint32_t (&ab)[2], int mi, int t) {
  return *(const lds_bf16x8*)((lds_cchar*)(uintptr_t)ab[t] + mi * 32 * 64);
}

// One stage (2 k-steps x 2 x NN MFMAs: this wave's 2 row tiles by its NN column tiles) on the
// current buffer, with the stage boundary inside it. Operands rotate through registers: the B
// read for k-step 1 of column tile c follows the two MFMAs of k-step 0 that consume it, and
// the A operands of k-step 1 are read at the start of k-step 0. Then every LDS read and all
// but `keep` of this wave's loads (those of the next stage included) are waited for and the
// block synchronises, and k-step 1 runs from registers while the next buffer's k-step 0
// operands are read and, when `load2`, the loads of the stage at K offset k2 are issued into
// the current buffer, which no wave reads any more. The matrix pipe is thus never left
// waiting for a whole LDS round trip at a stage boundary.
template <int NN, bool BT>
__device__ __forceinline__ void stage(const uint32_t (&ab)[2], const uint32_t (&bb)[4],
                                      const uint32_t (&abn)[2], const uint32_t (&bbn)[4],
                                      f32x16 (&acc)[2][8], bf16x8& a0, bf16x8& a1, bf16x8 (&b)[8],
                                      const Loader& ld, int64_t k2, bool load2, uint32_t sa,
                                      int wv, int keep) {
  {
    const bf16x8 n0 = read_a(ab, 0, 1), n1 = read_a(ab, 1, 1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int c = 0; c < NN; ++c) {
      acc[0][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b[c], acc[0][c], 0, 0, 0);
      acc[1][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b[c], acc[1][c], 0, 0, 0);
      b[c] = read_b_any<BT>(bb, c, 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    a0 = n0;
    a1 = n1;
  }
  wait_keep(keep);
  block_barrier();
  __builtin_amdgcn_sched_barrier(0);
  const bf16x8 n0 = read_a(abn, 0, 0), n1 = read_a(abn, 1, 0);
  __builtin_amdgcn_sched_barrier(0);
  const int64_t bk = k2 * ld.b_row_bytes;
#pragma unroll
  for (int c = 0; c < NN; ++c) {
    acc[0][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b[c], acc[0][c], 0, 0, 0);
    acc[1][c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b[c], acc[1][c], 0, 0, 0);
    b[c] = read_b_any<BT>(bbn, c, 0);
    if (load2) {
#pragma unroll
      for (int d = c * (8 / NN); d < (c + 1) * (8 / NN); ++d) load_one<BT>(ld, k2, bk, sa, wv, d);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  a0 = n0;
  a1 = n1;
}

// Wave layouts of a tile (NN = column tiles of 32 per wave):
//   NN = 8: wave w computes rows 64 w .. + 63, all 256 columns (any tile);
//   NN = 4: rows 64 (w % 2) .. + 63, columns 128 (w / 2) .. + 127 (tiles of at most 128 rows);
//   NN = 2: rows 0 .. 63, columns 64 w .. + 63 (tiles of at most 64 rows).
// A tile with fewer rows thus costs fewer MFMAs per wave, not idle waves. The read bases of
// one buffer for this wave: A rows start at the wave's first row; B column tile j of the wave
// is tile c = first + j of the block, read at bases[c % 4] + 256 bytes * (c / 4).
template <int NN>
__device__ __forceinline__ int wave_row0(int wv) {
  return NN == 8 ? 64 * wv : NN == 4 ? 64 * (wv & 1) : 0;
}
template <int NN>
__device__ __forceinline__ int wave_col_tile0(int wv) {
  return NN == 8 ? 0 : NN == 4 ? 4 * (wv >> 1) : 2 * wv;
}
template <int NN, bool BT>
__device__ __forceinline__ void unit_bases(uint32_t lds_a, uint32_t lds_b, const uint32_t (&aoff)[2],
                                           const uint32_t (&boff)[4], int wv, uint32_t (&ab)[2],
                                           uint32_t (&bb)[4]) {
  const uint32_t arow = (uint32_t)wave_row0<NN>(wv) * 64u;
  const int c0 = wave_col_tile0<NN>(wv);
  const uint32_t bhi = (uint32_t)(c0 >> 2) * 256u;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (i < 2) {
      ab[i] = lds_a + aoff[i] + arow;
      asm volatile("" : "+v"(ab[i]));
    }
    // column tile c0 + i of the block (only i < NN is read)
    const int q = (c0 + i) & 3;
    bb[i] = lds_b + (q == 0 ? boff[0] : q == 1 ? boff[1] : q == 2 ? boff[2] : boff[3]) + bhi;
    asm volatile("" : "+v"(bb[i]));
  }
  if (BT) {  // K-major B: A's offsets, from the wave's first column tile (32 columns of 64 B)
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      bb[t] = lds_b + aoff[t] + (uint32_t)c0 * 32u * 64u;
      asm volatile("" : "+v"(bb[t]));
    }
  }
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// Two floats to two bfloat16 (round to nearest even, one v_cvt_pk_bf16_f32), low half first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t));
}

// silu(g) = g / (1 + e^-g), with the hardware reciprocal (about 1 ulp).
__device__ __forceinline__ float silu_f(float g) {
  return g * __builtin_amdgcn_rcpf(1.f + __expf(-g));
}

// An accumulator, read into a VGPR where it is used. (Left to itself the compiler copies all
// 256 accumulators out of their AGPRs at the end of the K loop, which needs more VGPRs than
// there are; the spilled ones then cost scratch round trips that also wait for every store.)
__device__ __forceinline__ float acc_get(float a) {
  float r;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(a));
  return r;
}

// The value of lane l ^ 1.
__device__ __forceinline__ float swap_adjacent_lanes(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xf, 0xf, true));
}

template <int EPI, bool BT = false, bool KG = false, bool SAVE = false>
__global__ __launch_bounds__(kThreads, 1) void gemm_bf16_256_kernel(const GroupedGemm g, int nt) {
  constexpr bool kSwiGLU = EPI == EPI_SWIGLU;
  static_assert(!BT || EPI == EPI_NONE, "the K-major B mode has no epilogue");
  static_assert(!KG || (EPI == EPI_NONE && !BT), "the K-grouped mode has no epilogue");
  static_assert(!SAVE || EPI != EPI_NONE, "only an activation has pre-activations to store");
  __shared__ __align__(16) char sbuf[kNBuf * kBuf];
  __shared__ int s_unit[2];  // work positions of later units, by unit parity
  __shared__ int s_last;
  __shared__ int s_scan[kThreads / kWave][kScanWords];  // each wave's tile scan

  // One block per CU (gridDim.x blocks: a multiple of 8, at most kSplitSlots). Tiles that fill
  // whole waves of the blocks run over all of K. When the count leaves a partial last wave of
  // r tiles, those tiles are split along K into s parts (r * s <= blocks, each part an even
  // number of stages), so the tail is one short wave instead of a long, mostly idle one.
  // Block b runs on XCD b % 8. Each XCD owns a contiguous eighth of the whole tiles, then an
  // eighth of the split parts, and its blocks take them in order from the XCD's counter, so
  // the tiles an XCD runs at once are neighbours that share rows and columns in its L2, and a
  // block that finishes early simply takes the next one.
  const int b = blockIdx.x, nblk = gridDim.x;
  int total_main, total;  // tiles that are not short, all tiles (wave-uniform)
  {
    const TileScan sc = tile_scan(g.offsets, g.E, kBM, nt);
    scan_store(sc, s_scan[threadIdx.x >> 6]);
    total_main = __builtin_amdgcn_readfirstlane(sc.total_main);
    total = __builtin_amdgcn_readfirstlane(sc.total);
  }
  // every value that steers the loops is wave-uniform; saying so keeps them under scalar
  // control (a divergent trip count would make the compiler copy the accumulators)
  if (total == 0) return;
  const int nst_all = (int)(g.K / kBK);
  int full = total, r = 0, split = 1;
  if (g.split_ws && nblk <= kSplitSlots && total % nblk != 0) {
    full = total / nblk * nblk;
    r = total - full;
    split = min(kMaxSplit, nblk / r);
    // each part needs a multiple of kNBuf stages (like every unit: see the stage loop), and
    // enough of them (kMinPartStages) to pay for storing and adding its float32 partial
    while (split > 1 && (nst_all % split != 0 || nst_all / split < kMinPartStages ||
                         (nst_all / split) % kNBuf != 0))
      --split;
    if (split == 1) full = total;
  }
  // Short tiles last (see tile_of) when the split tail holds all of them.
  const bool short_last =
      split > 1 && total - total_main <= r;
  const int xcd = b & 7, per = nblk >> 3, jb = b >> 3;
  // Work positions: q * 8 + x stands for entry q of XCD x's list (its eighth of the whole
  // tiles, or of all tiles when nothing is split); -2: no whole tile is left anywhere; -1:
  // nothing. Entries j and per + j of its own XCD's list are block (xcd, j)'s first two units;
  // the XCD's counter hands out the rest of the list from 2 per on, in order, and a block whose
  // own list is used up takes entries of the other XCDs' lists (so every XCD ends at about the
  // same time). Each block's K part (at most one, r * s <= blocks) comes last and is its own:
  // taking parts from a queue would let one block take two while another, still busy with its
  // whole tiles, gets none.
  const int chunk = (total + 7) >> 3;  // list length per XCD when nothing is split
  const int F8 = full >> 3;            // whole tiles per XCD when the tail is split
  bool part_taken = false;
  auto unit_at = [&](int pos, int& L, int& ks) -> bool {
    ks = 0;
    L = 0;
    if (pos >= 0) {
      const int src = pos & 7, q = pos >> 3;
      if (split == 1) {
        L = src * chunk + q;
        return q < chunk && L < total;
      }
      if (q < F8) {
        L = src * F8 + q;
        return true;
      }
      // an own entry past the whole tiles: this block's K part
    } else if (pos != -2 || split == 1) {
      return false;
    }
    if (split == 1 || part_taken) return false;
    const int R8 = (r * split + 7) >> 3;
    const int u = xcd * R8 + jb;
    if (jb >= R8 || u >= r * split) return false;
    part_taken = true;
    L = full + u / split;
    ks = u % split;
    return true;
  };
  // The next work position from the counters (own XCD first), for thread 0 only.
  unsigned done_mask = 0;  // lists this thread has found used up
  auto grab = [&]() -> int {
    for (int d = 0; d < 8; ++d) {
      const int src = (xcd + d) & 7;
      if (done_mask & (1u << src)) continue;
      const int q = 2 * per + atomicAdd(g.queue + src, 1);
      const int lim = split == 1 ? min(chunk, total - src * chunk) : F8;
      if (q < lim) return q * 8 + src;
      done_mask |= 1u << src;
    }
    return split == 1 ? -1 : -2;
  };

  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t K = g.K, N = g.N;

  // Geometry of a unit (all wave-uniform).
  struct Unit {
    int L, ks, e, row0, rows, n_tile, parts, nst;
    int64_t kbeg;
    int64_t acol, brow;  // K-grouped: the group's first A column and first B row
  };
  auto geometry = [&](int L, int ks) {
    Unit u;
    u.L = L;
    u.ks = ks;
    // M-blocks for the weight gradients (16 to 56 M-tiles a group, all whole); the forward's
    // experts have a few M-tiles, the last often ragged, and keep them in one block
    tile_of(scan_load(s_scan[threadIdx.x >> 6], total_main, total), g.offsets, kBM, nt,
            KG ? kTileBlockM : INT_MAX, kTileBlockN, short_last, L, u.e, u.row0, u.rows, u.n_tile);
    u.e = __builtin_amdgcn_readfirstlane(u.e);
    u.row0 = __builtin_amdgcn_readfirstlane(u.row0);
    u.rows = __builtin_amdgcn_readfirstlane(u.rows);
    u.n_tile = __builtin_amdgcn_readfirstlane(u.n_tile);
    u.parts = L >= full ? split : 1;  // K parts of this tile
    u.nst = nst_all / u.parts;        // a multiple of 4: K % 128 == 0, and so are the parts
    u.kbeg = (int64_t)ks * u.nst * kBK;
    u.acol = 0;
    u.brow = 0;
    if (KG) {  // the group's own K range (a multiple of 128, never empty); nothing is split
      const int k0 = __builtin_amdgcn_readfirstlane(g.k_offsets[u.e]);
      const int k1 = __builtin_amdgcn_readfirstlane(g.k_offsets[u.e + 1]);
      u.nst = (k1 - k0) / kBK;
      u.kbeg = 0;
      u.acol = k0;
      u.brow = __builtin_amdgcn_readfirstlane(g.b_offsets[u.e]);
    }
    return u;
  };

  // A: instruction j of wave w fills tile rows 16 (4w + j) + lane / 4; its 16-byte chunk at
  // position lane % 4 is logical chunk (lane % 4) ^ ((row / 4) % 4), and (row / 4) % 4 =
  // lane / 16 % 4. Rows past the tile read row 0 of the expert block (valid memory; their
  // outputs are never stored). The source rows of a unit are fetched ahead
  // (`gather_rows`) and turned into addresses when its loads are about to be issued.
  auto gather_rows = [&](const Unit& u, int32_t (&src)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int rr = 16 * (4 * wv + j) + (lane >> 2);
      const int64_t gr = u.row0 + (rr < u.rows ? rr : 0);
      if (KG) {  // row m of the group's transposed operand
        src[j] = (int32_t)(gr - (int64_t)u.e * g.group_rows);
      } else if (g.a_gather) {  // a negative entry: an empty padded row (the zero row)
        const int32_t v = g.a_gather[gr];
        src[j] = v < 0 ? -1 : v / g.gather_div;
      } else {
        src[j] = (int32_t)gr;
      }
    }
  };
  auto make_loader = [&](const Unit& u, const int32_t (&src)[4]) {
    Loader ld;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = (lane & 3) ^ ((lane >> 4) & 3);
      ld.a[j] = (src[j] < 0 && g.a_zero)
                    ? (const char*)g.a_zero + (u.acol + 8 * c) * 2
                    : (const char*)g.A + ((int64_t)src[j] * g.lda + u.acol + 8 * c) * 2;
    }
    // B: instruction j of wave w fills K-rows 8w + 2j + lane / 32; position lane % 32 of the
    // K-row holds logical chunk (lane % 32) ^ (4 (K-row % 4)), K-row % 4 = 2 (j % 2) + lane / 32.
    const int64_t n0 = (int64_t)u.n_tile * (kSwiGLU ? kBN / 2 : kBN);
    ld.b_row_bytes = N * 2;
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const int c = (lane & 31) ^ (4 * ((2 * q + (lane >> 5)) & 3));
      int64_t col;
      const uint16_t* Wm;
      if (kSwiGLU) {
        const int ct = c >> 2;  // n-tile of 32: even -> W1, odd -> W3, same output columns
        Wm = (const uint16_t*)((ct & 1) ? g.B1 : g.B0);
        col = n0 + 32 * (ct >> 1) + 8 * (c & 3);
      } else {
        Wm = (const uint16_t*)g.B0;
        col = n0 + 8 * c;
      }
      const int krow = 8 * wv + (lane >> 5);
      const int64_t brow0 = KG ? u.brow * N : (int64_t)u.e * K * N;
      ld.b[q] = (const char*)(Wm + brow0 + (int64_t)krow * N + (col < N ? col : 0));
    }
    if (BT) {
      // K-major B ((N, K) per expert): instruction j of wave w fills columns 16 (4w + j) +
      // lane / 4 like A's rows (columns past N read column 0; their outputs are never stored)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int64_t col = n0 + 16 * (4 * wv + j) + (lane >> 2);
        const int c = (lane & 3) ^ ((lane >> 4) & 3);
        ld.bt[j] = (const char*)((const uint16_t*)g.B0 +
                                 ((int64_t)u.e * N + (col < N ? col : 0)) * K + 8 * c);
      }
    }
    return ld;
  };

  // Operand read offsets within a stage buffer: A for row lane % 32 (the wave's first row and
  // the row tile are added as constants), B for the block's column tiles 0..3 (see
  // `unit_bases`).
  uint32_t aoff[2], boff[4];
  {
    const int rr = lane & 31;  // + 32 mi
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int chunk = (2 * t + (lane >> 5)) ^ ((rr >> 2) & 3);
      aoff[t] = (uint32_t)(rr * 64 + chunk * 16);
    }
    const int gq = lane >> 4, Lq = lane & 15;
    const int krow = 8 * (gq >> 1) + (Lq >> 2);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int chunk = (4 * c + 2 * (gq & 1) + ((Lq & 3) >> 1)) ^ (4 * (Lq >> 2));
      boff[c] = (uint32_t)(krow * 512 + chunk * 16 + 8 * (Lq & 1));
    }
  }
  const uint32_t lbase = lds_addr(sbuf);


  int L0, ks0;
  if (unit_at(jb * 8 + xcd, L0, ks0)) {
    Unit cu = geometry(L0, ks0);
    Loader ld;
    {
      int32_t src[4];
      gather_rows(cu, src);
      ld = make_loader(cu, src);
    }
    // The first unit's first kNBuf stages; every later unit's are loaded by the last kNBuf
    // stages of the unit before it.
#pragma unroll
    for (int q = 0; q < kNBuf; ++q)
      load_stage<BT>(ld, cu.kbeg + (int64_t)q * kBK, lbase + q * kBuf, wv);

    uint16_t* C = (uint16_t*)g.C;
    for (int i = 0;; ++i) {
      int Ln, ksn;
      // (the first unit's successor is fixed; later ones were published through LDS)
      const int qn =
          i == 0 ? (per + jb) * 8 + xcd : __builtin_amdgcn_readfirstlane(s_unit[(i + 1) & 1]);
      const bool has_next = unit_at(qn, Ln, ksn);

      f32x16 acc[2][8];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int c = 0; c < 8; ++c)
#pragma unroll
          for (int v = 0; v < 16; ++v) acc[mi][c][v] = 0.f;

      if (i == 0) {
        wait_keep((kNBuf - 1) * 8);
        block_barrier();
      }
      // The unit after next (taken now so that its atomic is not waited for at this barrier),
      // and the next unit's source rows: both are in flight while this unit computes.
      int after_next = -1;
      if (tid == 0 && has_next && Ln < full) after_next = grab();  // none after a K part
      Unit nx = cu;
      int32_t nsrc[4];
      if (has_next) {
        nx = geometry(Ln, ksn);
        gather_rows(nx, nsrc);
      }
      // The wave layout follows the tile's rows (K parts always use the full layout, since
      // their partial tiles are laid out by it).
      const int shape = (cu.parts > 1 || cu.rows > 128) ? 0 : (cu.rows > 64 ? 1 : 2);
      auto run = [&](auto nn_tag) {
        constexpr int NN = decltype(nn_tag)::value;
        uint32_t vab[2], vbb[4];  // read bases in buffer 0
        unit_bases<NN, BT>(lbase, lbase + kHalf, aoff, boff, wv, vab, vbb);
        bf16x8 a0 = read_a(vab, 0, 0), a1 = read_a(vab, 1, 0), bq[8];
#pragma unroll
        for (int c = 0; c < NN; ++c) bq[c] = read_b_any<BT>(vbb, c, 0);
        const int nst = cu.nst;
        const int64_t kbeg = cu.kbeg;
        // One stage on buffer CI (the next one is CI + 1 mod kNBuf): loads through loader LDR
        // of the stage at K offset KL go into buffer CI when LOAD; KEEP of this wave's loads may
        // stay in flight at the stage's barrier. Every unit has a multiple of kNBuf stages, so
        // each starts in buffer 0 and the loop below runs kNBuf stages per trip with the buffer
        // offsets as constants (they end up in the DS instructions' offset fields). (A macro,
        // not a lambda: captured operand arrays would live in scratch memory.)
#define MOE_STAGE(CI, LDR, KL, LOAD, KEEP)                                                  \
  {                                                                                         \
    constexpr uint32_t kco = (CI) * kBuf, kno = ((CI) + 1) % kNBuf * kBuf;                  \
    uint32_t ab[2], bb[4], abn[2], bbn[4];                                                  \
    _Pragma("unroll") for (int t = 0; t < 2; ++t) {                                         \
      ab[t] = vab[t] + kco;                                                                 \
      abn[t] = vab[t] + kno;                                                                \
    }                                                                                       \
    _Pragma("unroll") for (int c = 0; c < 4; ++c) {                                         \
      bb[c] = vbb[c] + kco;                                                                 \
      bbn[c] = vbb[c] + kno;                                                                \
    }                                                                                       \
    stage<NN, BT>(ab, bb, abn, bbn, acc, a0, a1, bq, LDR, KL, LOAD, lbase + kco, wv, KEEP); \
  }
        static_assert(kNBuf == 4, "the stage loop is written out for four buffers");
        for (int s = 0; s + kNBuf < nst; s += kNBuf) {
          MOE_STAGE(0, ld, kbeg + (int64_t)(s + 4) * kBK, true, kKeep)
          MOE_STAGE(1, ld, kbeg + (int64_t)(s + 5) * kBK, true, kKeep)
          MOE_STAGE(2, ld, kbeg + (int64_t)(s + 6) * kBK, true, kKeep)
          MOE_STAGE(3, ld, kbeg + (int64_t)(s + 7) * kBK, true, kKeep)
        }
        // Publish the unit after next (its slot was last read before this unit's barriers),
        // then let the last kNBuf stages load the next unit's first kNBuf. With no next unit
        // those stages load nothing, so fewer loads are left to keep in flight.
        if (tid == 0) s_unit[i & 1] = after_next;
        if (has_next) ld = make_loader(nx, nsrc);
        MOE_STAGE(0, ld, nx.kbeg, has_next, has_next ? kKeep : 16)
        MOE_STAGE(1, ld, nx.kbeg + kBK, has_next, has_next ? kKeep : 8)
        MOE_STAGE(2, ld, nx.kbeg + 2 * kBK, has_next, has_next ? kKeep : 0)
        MOE_STAGE(3, ld, nx.kbeg + 3 * kBK, has_next, has_next ? kKeep : 0)
#undef MOE_STAGE

        const int row0 = cu.row0, rows = cu.rows, parts = cu.parts, L = cu.L, ks = cu.ks;
        const int64_t n0 = (int64_t)cu.n_tile * (kSwiGLU ? kBN / 2 : kBN);  // first output col
        const int wr0 = wave_row0<NN>(wv), wc0 = wave_col_tile0<NN>(wv);
        // 32x32 accumulator layout: lane l holds column l % 32, rows 8*(v/4) + 4*(l/32) + v%4.
        // Output store of this wave's rows: lanes l and l ^ 1 hold adjacent columns of the same
        // rows. For each pair of rows (v0, v0 + 1) they swap one value, so the even lane stores
        // columns (c, c + 1) of row v0 and the odd lane the same two columns of row v0 + 1: one
        // 4-byte store per two outputs. cq is the output column of the lanes' 32-column tile.
        const bool odd = lane & 1;
        const int lrow = wr0 + 4 * (lane >> 5) + (odd ? 1 : 0);
        const int colp = (lane & 31) & ~1;
        const int64_t lofs = (int64_t)(row0 + lrow) * N + n0 + colp;
        uint16_t* lp = C + lofs;
        // optional stores of the pre-activations (the up GEMM's x W1 and x W3), same layout as C
        uint16_t* const pa = (uint16_t*)g.pre_a;
        uint16_t* const pb = (uint16_t*)g.pre_b;
        const int ccol0 = 32 * (kSwiGLU ? wc0 / 2 : wc0);  // first output column of the wave
        const int ccols = 32 * (kSwiGLU ? NN / 2 : NN);
        const bool whole = wr0 + 64 <= rows && n0 + ccol0 + ccols <= N;
        auto put_at = [&](uint16_t* base, int mi, int v0, int cq, float x0, float x1) {
          const float recv = swap_adjacent_lanes(odd ? x0 : x1);
          const uint32_t pk = odd ? pack_bf16x2(recv, x1) : pack_bf16x2(x0, recv);
          const int dr = 32 * mi + 8 * (v0 >> 2) + (v0 & 3);
          if (whole || (lrow + dr < rows && n0 + cq + colp < N))
            *(uint32_t*)(base + lofs + (int64_t)dr * N + cq) = pk;
        };
        auto put = [&](int mi, int v0, int cq, float x0, float x1) { put_at(C, mi, v0, cq, x0, x1); };
        if (parts == 1) {
          if (wr0 < rows) {  // a whole tile: store this wave's part from the accumulators
            // Rows outer: one 64-bit add per row (the lane's row pointer), then the row's
            // column tiles at immediate offsets. The bounds are tested only in a tile at an edge
            // of C (a scalar branch picks the copy of the loop).
            uint16_t* const pal = SAVE ? pa + lofs : nullptr;
            uint16_t* const pbl = SAVE ? pb + lofs : nullptr;
            auto store2 = [&](uint16_t* ptr, float x0, float x1, bool ok) {
              const float recv = swap_adjacent_lanes(odd ? x0 : x1);
              const uint32_t pk = odd ? pack_bf16x2(recv, x1) : pack_bf16x2(x0, recv);
              if (ok) *(uint32_t*)ptr = pk;
            };
            auto store_tile = [&](auto chk_tag) {
              constexpr bool kChk = decltype(chk_tag)::value;
#pragma unroll
              for (int mi = 0; mi < 2; ++mi)
#pragma unroll
                for (int v0 = 0; v0 < 16; v0 += 2) {
                  const int dr = 32 * mi + 8 * (v0 >> 2) + (v0 & 3);
                  const int64_t ro = (int64_t)dr * N;
                  const bool rok = !kChk || lrow + dr < rows;
#pragma unroll
                  for (int q = 0; q < (kSwiGLU ? NN / 2 : NN); ++q) {
                    const int cq = ccol0 + 32 * q;
                    const bool ok = !kChk || (rok && n0 + cq + colp < N);
                    float x0, x1;
                    if (kSwiGLU) {  // gate in the wave's column tile 2q, up in 2q + 1
                      const float g0 = acc_get(acc[mi][2 * q][v0]);
                      const float g1 = acc_get(acc[mi][2 * q][v0 + 1]);
                      const float u0 = acc_get(acc[mi][2 * q + 1][v0]);
                      const float u1 = acc_get(acc[mi][2 * q + 1][v0 + 1]);
                      x0 = silu_f(g0) * u0;
                      x1 = silu_f(g1) * u1;
                      if constexpr (SAVE) {
                        store2(pal + ro + cq, g0, g1, ok);
                        store2(pbl + ro + cq, u0, u1, ok);
                      }
                    } else {
                      x0 = acc_get(acc[mi][q][v0]);
                      x1 = acc_get(acc[mi][q][v0 + 1]);
                      if (EPI == EPI_RELU) {
                        if constexpr (SAVE) store2(pal + ro + cq, x0, x1, ok);
                        x0 = fmaxf(x0, 0.f);
                        x1 = fmaxf(x1, 0.f);
                      }
                    }
                    store2(lp + ro + cq, x0, x1, ok);
                  }
                }
            };
            if (whole)
              store_tile(std::false_type{});
            else
              store_tile(std::true_type{});
          }
        } else if constexpr (NN == 8) {
          // A K part: store the float32 partial tile (each lane's accumulators, 16 bytes at a
          // time, in a lane-interleaved layout), then take a ticket; the part that takes the last
          // ticket adds all parts in part order and stores the tile. The sum order is fixed, so
          // the result does not depend on which part finishes last.
          float* slots = g.split_ws + (int64_t)(L - full) * parts * kSplitSlotFloats;
          if (wr0 < rows) {
            float* mine = slots + (int64_t)ks * kSplitSlotFloats;
            // group (wv, mi, c) of 16 accumulators: 4 KB at a wave-uniform base, lane l's 16-byte
            // chunk v4 at +1 KB * v4 + 16 l (so every store is base + one lane offset + a const)
            const uint32_t lane_off = (uint32_t)lane * 16u;
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
#pragma unroll
              for (int c = 0; c < 8; ++c) {
                char* gb = (char*)mine + (int64_t)((wv * 2 + mi) * 8 + c) * 4096;
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4)
                  *(f32x4*)(gb + v4 * 1024 + lane_off) =
                      f32x4{acc_get(acc[mi][c][4 * v4]), acc_get(acc[mi][c][4 * v4 + 1]),
                            acc_get(acc[mi][c][4 * v4 + 2]), acc_get(acc[mi][c][4 * v4 + 3])};
              }
          }
          __threadfence();
          __syncthreads();
          if (tid == 0) s_last = atomicAdd(&g.split_ctr[L - full], 1) == parts - 1;
          __syncthreads();
          if (s_last) {
            __threadfence();
            if (tid == 0) g.split_ctr[L - full] = 0;  // ready for the next launch
            if (wr0 < rows) {
              // Every part (this one included) has stored its partial: add them in part order,
              // 16 coalesced bytes (4 rows of one column) per lane and part at a time, and store
              // the rows.
              const uint32_t lane_off = (uint32_t)lane * 16u;
              for (int mi = 0; mi < 2; ++mi)
                for (int v4 = 0; v4 < 4; ++v4) {
                  // every part of this row group's 8 column tiles, all loads issued before any
                  // is used; then added in part order
                  f32x4 pv[kMaxSplit][8];
#pragma unroll
                  for (int q = 0; q < kMaxSplit; ++q)
#pragma unroll
                    for (int c = 0; c < 8; ++c)
                      if (q < parts)
                        pv[q][c] = *(const f32x4*)((const char*)slots +
                                                   (int64_t)((wv * 2 + mi) * 8 + c) * 4096 +
                                                   v4 * 1024 + q * kSplitSlotFloats * 4 + lane_off);
                  f32x4 t[8];
#pragma unroll
                  for (int c = 0; c < 8; ++c) {
                    t[c] = pv[0][c];
#pragma unroll
                    for (int q = 1; q < kMaxSplit; ++q)
                      if (q < parts) t[c] += pv[q][c];
                  }
                  // rows 8 v4 + 4 (lane / 32) + i4 of the lanes' columns: accumulator rows
                  // v = 4 v4 + i4, stored as the pairs (v, v + 1) like a whole tile
                  if (kSwiGLU) {
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                      const f32x4 gt = t[2 * q], up = t[2 * q + 1];
#pragma unroll
                      for (int i4 = 0; i4 < 4; i4 += 2) {
                        put(mi, 4 * v4 + i4, 32 * q, silu_f(gt[i4]) * up[i4],
                            silu_f(gt[i4 + 1]) * up[i4 + 1]);
                        if constexpr (SAVE) {
                          put_at(pa, mi, 4 * v4 + i4, 32 * q, gt[i4], gt[i4 + 1]);
                          put_at(pb, mi, 4 * v4 + i4, 32 * q, up[i4], up[i4 + 1]);
                        }
                      }
                    }
                  } else {
#pragma unroll
                    for (int c = 0; c < 8; ++c) {
                      f32x4 x = t[c];
                      if (EPI == EPI_RELU) {
                        if constexpr (SAVE)
#pragma unroll
                          for (int i4 = 0; i4 < 4; i4 += 2)
                            put_at(pa, mi, 4 * v4 + i4, 32 * c, x[i4], x[i4 + 1]);
#pragma unroll
                        for (int i4 = 0; i4 < 4; ++i4) x[i4] = fmaxf(x[i4], 0.f);
                      }
#pragma unroll
                      for (int i4 = 0; i4 < 4; i4 += 2) put(mi, 4 * v4 + i4, 32 * c, x[i4], x[i4 + 1]);
                    }
                  }
                }
            }
          }
        }
      };
      if (shape == 0)
        run(std::integral_constant<int, 8>{});
      else if (shape == 1)
        run(std::integral_constant<int, 4>{});
      else
        run(std::integral_constant<int, 2>{});
      if (!has_next) break;
      cu = nx;
    }
  }
  // The last block to finish resets the queue for the next launch (every block has taken its
  // last position by then).
  if (tid == 0) {
    __threadfence();
    if (atomicAdd(g.queue + 8, 1) == nblk - 1) {
#pragma unroll
      for (int x = 0; x < 8; ++x) g.queue[x] = 0;
      g.queue[8] = 0;
    }
  }
}

__global__ void zero_tickets_kernel(int32_t* __restrict__ p, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) p[i] = 0;
}

}  // namespace

hipError_t launch_zero_tickets(int32_t* tickets, int n, hipStream_t s) {
  hipLaunchKernelGGL(zero_tickets_kernel, dim3(1), dim3(256), 0, s, tickets, n);
  return hipGetLastError();
}

int device_split_cus() {
  static int cache[64] = {0};  // per device: 0 unknown, -1 not usable, else the CU count
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    n = n < kSplitSlots ? n : kSplitSlots;
    cache[dev] = (n >= 8 && n % 8 == 0) ? n : -1;
  }
  return cache[dev] > 0 ? cache[dev] : 0;
}

// A K split needs at least two parts of kMinPartStages stages each; its parts never outnumber
// the launch's blocks (at most one a block), whose count is capped by the tile bound (rounded up
// to 8) and by kSplitSlots.
int64_t gemm_bf16_split_slots(int64_t max_rows, int E, int64_t K, int64_t N, bool swiglu) {
  if (K % 128 != 0 || K / kBK < 2 * kMinPartStages) return 0;
  const int64_t mt_max = (max_rows + kBM - 1) / kBM + E;
  const int64_t cols = swiglu ? kBN / 2 : kBN;
  const int64_t tiles = (mt_max * ((N + cols - 1) / cols) + 7) / 8 * 8;
  return tiles < kSplitSlots ? tiles : kSplitSlots;
}

hipError_t launch_grouped_gemm_bf16_256(const GroupedGemm& g_in, hipStream_t s) {
  GroupedGemm g = g_in;
  // A K split needs at least two parts of kMinPartStages stages each; below that the split
  // path (and its ticket reset) is skipped altogether. K-grouped products are never split.
  if (g.k_grouped || g.K / kBK < 2 * kMinPartStages) {
    g.split_ws = nullptr;
    g.split_ctr = nullptr;
  }
  const int64_t mt_max = (g.max_rows + kBM - 1) / kBM + g.E;
  const int64_t cols = (g.epilogue == EPI_SWIGLU) ? kBN / 2 : kBN;
  const int64_t nt = (g.N + cols - 1) / cols;
  // One block per CU (a multiple of 8, at most kSplitSlots, the split parts' slot count), or
  // fewer when there are fewer tiles than that. The kernel takes its block count as the
  // width of a wave of tiles.
  int64_t G = g.ncu >= 8 ? g.ncu : kSplitSlots;
  if (G > kSplitSlots) G = kSplitSlots;
  G = G / 8 * 8;
  const int64_t tiles_max = (mt_max * nt + 7) / 8 * 8;
  if (G > tiles_max) G = tiles_max;
  // (the parts of a split never outnumber the blocks: a workspace with fewer slots is not used)
  if (g.split_ws && G > g.split_slots) {
    g.split_ws = nullptr;
    g.split_ctr = nullptr;
  }
  const dim3 grid((unsigned)G);
  // The start/stop events (if any) are recorded by the kernel's own dispatch, so timing adds
  // no packets, and no gaps, to the stream.
  if (g.b_kmajor) {
    hipExtLaunchKernelGGL((gemm_bf16_256_kernel<EPI_NONE, true>), grid, dim3(kThreads), 0, s,
                          g.ev_start, g.ev_stop, 0, g, (int)nt);
    return hipGetLastError();
  }
  if (g.k_grouped) {
    hipExtLaunchKernelGGL((gemm_bf16_256_kernel<EPI_NONE, false, true>), grid, dim3(kThreads), 0,
                          s, g.ev_start, g.ev_stop, 0, g, (int)nt);
    return hipGetLastError();
  }
  switch (g.epilogue) {
    case EPI_NONE:
      hipExtLaunchKernelGGL(gemm_bf16_256_kernel<EPI_NONE>, grid, dim3(kThreads), 0, s,
                            g.ev_start, g.ev_stop, 0, g, (int)nt);
      break;
    case EPI_RELU:
      if (g.pre_a)
        hipExtLaunchKernelGGL((gemm_bf16_256_kernel<EPI_RELU, false, false, true>), grid,
                              dim3(kThreads), 0, s, g.ev_start, g.ev_stop, 0, g, (int)nt);
      else
        hipExtLaunchKernelGGL(gemm_bf16_256_kernel<EPI_RELU>, grid, dim3(kThreads), 0, s,
                              g.ev_start, g.ev_stop, 0, g, (int)nt);
      break;
    default:
      if (g.pre_a)
        hipExtLaunchKernelGGL((gemm_bf16_256_kernel<EPI_SWIGLU, false, false, true>), grid,
                              dim3(kThreads), 0, s, g.ev_start, g.ev_stop, 0, g, (int)nt);
      else
        hipExtLaunchKernelGGL(gemm_bf16_256_kernel<EPI_SWIGLU>, grid, dim3(kThreads), 0, s,
                              g.ev_start, g.ev_stop, 0, g, (int)nt);
      break;
  }
  return hipGetLastError();
}

}  // namespace moe
