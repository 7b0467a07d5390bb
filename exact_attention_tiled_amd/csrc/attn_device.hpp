// attn_device.hpp - device building blocks of the exact tiled attention kernels (gfx950).
//
// Everything here is CDNA4-specific: 64-lane wavefronts, the 32x32 MFMA accumulator
// layout, LDS transpose reads, and XCD round-robin workgroup dispatch.
//
// MFMA 32x32 accumulator layout (measured on gfx950 for v_mfma_f32_32x32x16_bf16 and
// v_mfma_f32_32x32x2_f32): lane l, register r holds C[row][col] with
//     col = l % 32,   row = 8 * (r / 4) + 4 * (l / 32) + (r % 4).
// Operands of 32x32x16 bf16: lane l holds A[l % 32][8 * (l / 32) + t] and
// B[8 * (l / 32) + t][l % 32] for t = 0..7. Operands of 32x32x2 f32: lane l holds
// A[l % 32][l / 32] and B[l / 32][l % 32].
//
// The forward computes S^T = K Q^T (rows = keys, columns = queries), so after the QK^T
// contraction every lane owns ONE query (column l % 32) and 16 of the 32 keys of a block:
// the softmax row statistics are per-lane values plus one exchange with lane l ^ 32, and
// the P^T operand of the following O^T = V^T P^T contraction is already in registers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) int i32x4;
typedef __attribute__((ext_vector_type(2))) int i32x2;
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int WAVE = 64;
constexpr int LDS_BYTES = 160 * 1024;  // per workgroup on gfx950
constexpr float LOG2E = 1.4426950408889634f;
constexpr float LN2 = 0.6931471805599453f;
constexpr int MASK_NONE = 0;
constexpr int MASK_TOP_LEFT = 1;
constexpr int MASK_BOTTOM_RIGHT = 2;

__device__ __forceinline__ float neg_inf() { return -__builtin_inff(); }

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Value of the same register in lane l ^ 32 (the other half of the wave).
__device__ __forceinline__ float swap_halves(float x) {
  return __shfl_xor(x, 32);
}

// max / sum of x over lanes l and l ^ 32, in VALU only: v_permlane32_swap(x, x) yields the
// low half and the high half of x, each replicated to both halves of the wave.
__device__ __forceinline__ float max_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------------------
// Mask unit. Sequence geometry comes from cu_seqlens; positions are always in-sequence
// (0-based), never packed offsets. `off` is the alignment shift of the causal diagonal:
// 0 for top-left, len_k - len_q for bottom-right.
// ---------------------------------------------------------------------------------------
struct SeqGeom {
  int q_start, k_start;  // packed offsets of the sequence's first query / key token
  int len_q, len_k;
  int off;
};

// Values the whole workgroup shares but the compiler cannot prove uniform (they come from
// vector loads of cu_seqlens). Marking them uniform keeps address and descriptor
// arithmetic in scalar registers.
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Geometry of sequence s, which may differ from lane to lane.
__device__ __forceinline__ SeqGeom load_geom_lane(const int32_t* cu_q, const int32_t* cu_k, int s,
                                                  int mode) {
  SeqGeom g;
  g.q_start = cu_q[s];
  g.k_start = cu_k[s];
  g.len_q = cu_q[s + 1] - g.q_start;
  g.len_k = cu_k[s + 1] - g.k_start;
  g.off = (mode == MASK_BOTTOM_RIGHT) ? g.len_k - g.len_q : 0;
  return g;
}

// Geometry of sequence s when s is the same for the whole workgroup.
__device__ __forceinline__ SeqGeom load_geom(const int32_t* cu_q, const int32_t* cu_k, int s,
                                             int mode) {
  SeqGeom g = load_geom_lane(cu_q, cu_k, s, mode);
  g.q_start = uniform(g.q_start);
  g.k_start = uniform(g.k_start);
  g.len_q = uniform(g.len_q);
  g.len_k = uniform(g.len_k);
  g.off = uniform(g.off);
  return g;
}

// Key positions [lo, hi) visible from query position pq (none when hi <= lo). With
// end = pq + off the aligned diagonal: every key of the sequence without a causal mode;
// keys up to end with one; and only the `window` most recent of those, (end - window, end],
// with a window. Keys at or beyond len_k (out-of-range tile lanes) are never visible.
__device__ __forceinline__ void key_interval(int pq, const SeqGeom& g, int mode, int window,
                                             int& lo, int& hi) {
  const int end = pq + g.off;
  hi = mode == MASK_NONE ? g.len_k : min(g.len_k, end + 1);
  lo = (mode != MASK_NONE && window > 0) ? end - window + 1 : 0;
}

// Is key position pk >= 0 visible from query position pq? Branch-free on purpose: callers
// turn the result into a select, never into a divergent conditional store.
__device__ __forceinline__ bool pair_allowed(int pq, int pk, const SeqGeom& g, int mode,
                                             int window) {
  int lo, hi;
  key_interval(pq, g, mode, window, lo, hi);
  return (pk >= lo) & (pk < hi);
}

// Per-lane exclusion for NK 32-key blocks in accumulator layout (register r of block kb
// holds key kpos0 + 32 kb + 8 (r / 4) + 4 (l / 32) + r % 4 of this lane's query pq):
// disallowed entries become -inf. lo <= pk < hi is one unsigned compare of pk - lo against
// hi - lo, with pk - lo = base + (a compile-time constant per register).
template <int NK>
__device__ __forceinline__ void mask_blocks(f32x16 (&s)[NK], int pq, int kpos0, const SeqGeom& g,
                                            int mode, int window, int lane) {
  int lo, hi;
  key_interval(pq, g, mode, window, lo, hi);
  const int base = kpos0 + 4 * (lane >> 5) - lo;
  const unsigned width = hi > lo ? (unsigned)(hi - lo) : 0u;
#pragma unroll
  for (int kb = 0; kb < NK; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const unsigned x = (unsigned)(base + 32 * kb + 8 * (r >> 2) + (r & 3));
      s[kb][r] = x < width ? s[kb][r] : neg_inf();
    }
}

// Key positions [lo, hi) that any query position in [p0, p1) may see (p1 > p0).
__device__ __forceinline__ void visible_keys(int p0, int p1, const SeqGeom& g, int mode,
                                             int window, int& lo, int& hi) {
  if (mode == MASK_NONE) {
    lo = 0;
    hi = g.len_k;
    return;
  }
  hi = min(g.len_k, p1 + g.off);  // largest visible key is (p1 - 1) + off
  lo = window > 0 ? max(0, p0 + g.off - window + 1) : 0;
  if (hi < lo) hi = lo;
}

// Stages of BN keys that query rows [p0, p1) visit: stage i covers key positions
// [kstart + i BN, kstart + (i + 1) BN); nst = 0 when no key is visible.
__device__ __forceinline__ void stage_range(int p0, int p1, const SeqGeom& g, int mode,
                                            int window, int bn, int& kstart, int& nst) {
  int klo, khi;
  visible_keys(p0, p1, g, mode, window, klo, khi);
  kstart = (klo / bn) * bn;
  nst = khi > klo ? (khi - kstart + bn - 1) / bn : 0;
}

// Classification of a (query positions [p0,p1)) x (key positions [k0,k1)) block:
// 0 = no pair allowed, 1 = some pairs (per-lane test needed), 2 = every pair allowed.
__device__ __forceinline__ int block_class(int p0, int p1, int k0, int k1, const SeqGeom& g,
                                           int mode, int window) {
  if (p1 <= p0 || k0 >= g.len_k || k1 <= k0) return 0;
  if (mode != MASK_NONE) {
    if (k0 > p1 - 1 + g.off) return 0;                              // all keys in the future
    if (window > 0 && k1 - 1 <= p0 + g.off - window) return 0;      // all keys out of window
  }
  if (k1 > g.len_k) return 1;
  if (mode == MASK_NONE) return 2;
  if (k1 - 1 > p0 + g.off) return 1;
  if (window > 0 && k0 <= p1 - 1 + g.off - window) return 1;
  return 2;
}

// Split-K classification of one wave's KBW 32-key blocks at key position kw0 of a stage,
// rows [rlo, rhi) of the group's G * len_q (position, head) rows, chunk keys [klo, khi):
// returns the block class (0: the wave skips the stage) and sets clip when some keys of the
// blocks lie outside the chunk (they belong to a neighbouring chunk's partial).
template <int KBW>
__device__ __forceinline__ int splitk_stage_class(int kw0, int klo, int khi, int rlo, int rhi,
                                                  const SeqGeom& g, int G, int mode, int window,
                                                  bool& clip) {
  const int cw0 = max(kw0, klo), cw1 = min(kw0 + 32 * KBW, khi);
  clip = cw0 != kw0 || cw1 != kw0 + 32 * KBW;
  return (rhi <= rlo || cw1 <= cw0)
             ? 0
             : block_class(rlo / G, (rhi - 1) / G + 1, kw0, kw0 + 32 * KBW, g, mode, window);
}

// Split-K exclusion of keys outside the chunk for a classified stage (cls != 0); returns
// whether the stage then needs the per-lane test (mask_blocks) of disallowed pairs.
template <int KBW>
__device__ __forceinline__ bool splitk_stage_clip(f32x16 (&s)[KBW], int cls, bool clip, int kw0,
                                                  int klo, int khi, int lane) {
  if (clip) {
    const int cw0 = max(kw0, klo), cw1 = min(kw0 + 32 * KBW, khi);
    const int hg = lane >> 5;
#pragma unroll
    for (int i = 0; i < KBW; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kk = kw0 + 32 * i + 8 * (r >> 2) + 4 * hg + (r & 3);
        s[i][r] = ((kk >= cw0) & (kk < cw1)) ? s[i][r] : neg_inf();
      }
  }
  return cls == 1 || clip;
}

// Backward element tests (the same logical mask as the forward). dK/dV kernel: this lane's
// key has query interval [q_lo, q_lo + q_width) (query_interval); register r of a 32-query
// block starting at qa holds query qa + 8 (r / 4) + 4 (lane / 32) + r % 4.
struct KeyLaneTest {
  unsigned base, width;
  __device__ __forceinline__ KeyLaneTest(int qa, int cls, int hg, int q_lo, unsigned q_width)
      : base((unsigned)(qa + 4 * hg - q_lo)), width(cls == 2 ? 0xffffffffu : q_width) {}
  __device__ __forceinline__ bool ok(int r) const {
    return base + (unsigned)(8 * (r >> 2) + (r & 3)) < width;
  }
};
// dQ kernel: this lane's query has key interval [k_lo, k_lo + k_width) (key_interval);
// register r of 32-key block kb of a stage at k0 holds key k0 + 32 kb + 8 (r / 4) +
// 4 (lane / 32) + r % 4.
struct QueryLaneTest {
  unsigned base, width;
  __device__ __forceinline__ QueryLaneTest(int k0, int cls, int hg, int k_lo, unsigned k_width)
      : base((unsigned)(k0 + 4 * hg - k_lo)), width(cls == 2 ? 0xffffffffu : k_width) {}
  __device__ __forceinline__ bool ok(int kb, int r) const {
    return base + (unsigned)(32 * kb + 8 * (r >> 2) + (r & 3)) < width;
  }
};

// Sequence owning packed token t: largest s with cu[s] <= t, skipping empty sequences.
__device__ __forceinline__ int seq_of_token(const int32_t* cu, int num_seqs, int t) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------------------
// Varlen tile scheduler. Query tiles of BM rows start at each sequence's first token.
// Sequence s owns the slot range starting at floor(cu_q[s] / BM) + s; it uses its first
// ceil(len_q / BM) slots and the rest exit at once. Because floor(c / BM) + ceil(L / BM)
// <= floor((c + L) / BM) + 1, slot ranges never overlap, and floor(total_q / BM) +
// num_seqs slots cover every tile. The owner of a slot is found by binary search on
// cu_q, so the host never reads cu_seqlens and no prepass is needed.
// ---------------------------------------------------------------------------------------
template <int BM>
__device__ __forceinline__ int seq_of_slot(const int32_t* cu_q, int num_seqs, int slot) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (uniform(cu_q[mid]) / BM + mid <= slot) lo = mid; else hi = mid - 1;
  }
  return uniform(lo);
}

// Workgroups are handed to the 8 XCDs round-robin (block b runs on XCD b % 8). This maps
// the hardware block id to a logical work index so that consecutive logical items (the
// query tiles of one head and sequence, which read the same K/V) run on the same XCD and
// share its L2. Returns -1 for padding blocks.
__device__ __forceinline__ int xcd_logical_block(int b, int nlogical) {
  const int per = (nlogical + 7) >> 3;
  const int w = (b & 7) * per + (b >> 3);
  return w < nlogical ? w : -1;
}

// ---------------------------------------------------------------------------------------
// Dropout on the attention weights. The realisation must replay in the backward and
// across packings, so it is a function of logical indices only (Causal Mask and Ragged
// Sequence Layouts, section 6): the keep flag of (sequence index s, query head h,
// in-sequence query position i, key position j) is byte j % 4 of output word i % 4 of
// Philox4x32-10 at counter (i / 4, j / 4, h, s) under the 64-bit seed, kept iff the byte
// is at least thr = round(256 p). One generator call thus serves a 4 x 4 patch: the
// forward and dQ kernels (queries on lanes, 4 consecutive keys per register group) use one
// word of it, the dK/dV kernel (keys on lanes, 4 consecutive queries per group) one byte
// of each word.
// ---------------------------------------------------------------------------------------
struct DropoutSite {
  uint32_t seed_lo, seed_hi;
  uint32_t thr;    // 1..255 (0: no dropout; the kernels without it never read this)
  float scale;     // 1 / (1 - thr / 256)
  int s, h;        // sequence index, query head
};

// Philox4x32 with 10 rounds (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC'11): per round two 32 x 32 -> 64-bit products of counter words 0
// and 2 with the Philox multipliers, the new counter (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1,
// lo0), and the key advanced by the two Weyl constants before every round but the first.
__device__ __forceinline__ void philox4x32_10(uint32_t (&c)[4], uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint64_t p0 = (uint64_t)0xD2511F53u * c[0];
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c[2];
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c[1] ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c[3] ^ k1;
    c[1] = (uint32_t)p1;
    c[3] = (uint32_t)p0;
    c[0] = n0;
    c[2] = n2;
  }
}

// The patch of query positions 4 qp + 0..3 and key positions 4 kp + 0..3: w[a] holds
// query 4 qp + a, its byte b key 4 kp + b.
__device__ __forceinline__ void dropout_patch(const DropoutSite& d, int qp, int kp,
                                              uint32_t (&w)[4]) {
  w[0] = (uint32_t)qp;
  w[1] = (uint32_t)kp;
  w[2] = (uint32_t)d.h;
  w[3] = (uint32_t)d.s;
  philox4x32_10(w, d.seed_lo, d.seed_hi);
}

// The 4 lanes of an aligned quad share a query quad (forward, dQ) or a key quad (dK/dV), so
// the 4 patches a quad needs for the 4 register groups of a 32 x 32 block are computed
// once each: lane c of the quad generates the patch of group c, and every lane fetches the
// words it needs from the quad with DPP broadcasts (whole wave active).
template <int A>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, A * 0x55, 0xF, 0xF, false);
}

// Row form: keep[a] bit b = key 4 (kp0 + 2 a) + b for this lane's query pq (pq & 3 equals
// the lane's position in its quad). Group a covers keys 8 a + 4 (lane / 32) + 0..3 of a
// 32-key block, so kp0 = (block start + 4 (lane / 32)) / 4.
__device__ __forceinline__ void dropout_keep_rows4(const DropoutSite& d, int pq, int kp0,
                                                   uint32_t (&keep)[4]) {
  const int c = pq & 3;
  uint32_t w[4];
  dropout_patch(d, pq >> 2, kp0 + 2 * c, w);
  uint32_t x[4][4];  // x[a][v] = word v of group a's patch
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    x[0][v] = quad_bcast<0>(w[v]);
    x[1][v] = quad_bcast<1>(w[v]);
    x[2][v] = quad_bcast<2>(w[v]);
    x[3][v] = quad_bcast<3>(w[v]);
  }
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const uint32_t y = (c & 2) ? ((c & 1) ? x[a][3] : x[a][2]) : ((c & 1) ? x[a][1] : x[a][0]);
    uint32_t bits = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) bits |= (((y >> (8 * b)) & 0xFFu) >= d.thr ? 1u : 0u) << b;
    keep[a] = bits;
  }
}

// Column form: keep[a] bit v = query 4 (qp0 + 2 a) + v for this lane's key pk (pk & 3
// equals the lane's position in its quad). Group a covers queries 8 a + 4 (lane / 32) + 0..3
// of a 32-query block, so qp0 = (block start + 4 (lane / 32)) / 4.
__device__ __forceinline__ void dropout_keep_cols4(const DropoutSite& d, int qp0, int pk,
                                                   uint32_t (&keep)[4]) {
  const int c = pk & 3;
  uint32_t w[4];
  dropout_patch(d, qp0 + 2 * c, pk >> 2, w);
  const int sh = 8 * c;
#pragma unroll
  for (int a = 0; a < 4; ++a) keep[a] = 0;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    const uint32_t x0 = quad_bcast<0>(w[v]), x1 = quad_bcast<1>(w[v]);
    const uint32_t x2 = quad_bcast<2>(w[v]), x3 = quad_bcast<3>(w[v]);
    keep[0] |= (((x0 >> sh) & 0xFFu) >= d.thr ? 1u : 0u) << v;
    keep[1] |= (((x1 >> sh) & 0xFFu) >= d.thr ? 1u : 0u) << v;
    keep[2] |= (((x2 >> sh) & 0xFFu) >= d.thr ? 1u : 0u) << v;
    keep[3] |= (((x3 >> sh) & 0xFFu) >= d.thr ? 1u : 0u) << v;
  }
}

// ---------------------------------------------------------------------------------------
// Swizzled LDS tiles filled by buffer -> LDS DMA.
//
// A tile row r of ROWB bytes occupies [r * ROWB, (r + 1) * ROWB) with its 16-byte chunk c
// stored at slot c ^ key(r) (key below). The XOR spreads the chunks the MFMA operand reads
// touch together over different bank groups, so they avoid bank conflicts without padding (padding cannot be used: one DMA instruction writes 64 lanes x 16 bytes
// contiguously).
//
// buffer_load_dwordx4 ... lds writes lane l's 16 bytes to LDS at (wave-uniform base) +
// 16 l. Lane l of instruction i therefore fetches the global chunk that belongs at its
// fixed LDS slot. The buffer descriptor covers only the tile's valid rows, so rows past
// the sequence end (or the tensor end) are never read: the hardware range check returns
// zeros for them.
// ---------------------------------------------------------------------------------------
// gfx950 LDS serves 256 bytes per cycle (64 banks; measured with the bank-conflict
// counter). Row r's XOR key must therefore (i) give 16 consecutive rows 16 different
// 16-byte slots for one chunk (row-wise ds_read_b128 of the K operand, 16 lanes per cycle)
// and (ii) put the 4 rows read by half a wave of ds_read_b64_tr_b16 (4 chunks each) in 4
// different groups of 4 slots. For 256-byte rows the key is the 4x4 bit transpose of
// r mod 16; for 128-byte rows (two rows per 256-byte bank cycle) a 3-bit key of r / 2.
template <int ROWB>
__device__ __forceinline__ int swz_key(int row) {
  if (ROWB >= 256) return ((row & 3) << 2) | ((row >> 2) & 3);
  return (((row >> 1) & 1) << 2) | ((row >> 2) & 3);
}
template <int ROWB>
__device__ __forceinline__ int swz_chunk(int row, int chunk) { return chunk ^ swz_key<ROWB>(row); }

// Race exposure (test builds compiled with -DATTN_DEBUG_POISON_LDS). Every thread that is
// about to refill an LDS buffer first overwrites exactly the bytes it will refill with a
// finite sentinel (0x46EA46EA: about 3e4 read as fp32 and as each bf16 half), then refills
// them (program order keeps the sentinel from landing after the data). The refill only
// starts once the barrier that freed the buffer has passed, and readers of the new data
// only read after the barrier that publishes it; were either barrier missing, a wave would
// read the sentinel deterministically instead of the previous stage's plausible values.
// Release builds compile the poisoning to nothing.
constexpr int LDS_POISON = 0x46EA46EA;
__device__ __forceinline__ void poison16(char* lds) {
#if defined(ATTN_DEBUG_POISON_LDS)
  *reinterpret_cast<i32x4*>(lds) = i32x4{LDS_POISON, LDS_POISON, LDS_POISON, LDS_POISON};
#endif
}
__device__ __forceinline__ void poison8(char* lds) {
#if defined(ATTN_DEBUG_POISON_LDS)
  *reinterpret_cast<i32x2*>(lds) = i32x2{LDS_POISON, LDS_POISON};
#endif
}
__device__ __forceinline__ void poison4(float* lds) {
#if defined(ATTN_DEBUG_POISON_LDS)
  *lds = __int_as_float(LDS_POISON);
#endif
}
__device__ __forceinline__ void poison_done() {
#if defined(ATTN_DEBUG_POISON_LDS)
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#endif
}

// Cache-policy operand of the DMA loads. CPOL_NT sets the nontemporal (streaming) hint for
// data that one call reads exactly once: the split-K decode's K/V stream, which runs
// 4-11 % faster with it on gfx950 (measured). Tiles that other workgroups re-read (prefill
// and backward K/V, Q/dO) keep the default policy.
constexpr int CPOL_DEFAULT = 0;
constexpr int CPOL_NT = 2;

template <int ROWB, int ROWS, int NWAVES, int CPOL = CPOL_DEFAULT>
struct DmaStager {
  static constexpr int C = ROWB / 16;        // chunks per row
  static constexpr int RPI = 1024 / ROWB;    // rows per DMA instruction
  static constexpr int NINST = ROWS / RPI;   // instructions per tile
  static_assert(C >= 8 && NINST % NWAVES == 0, "tile shape");
  static constexpr int PER_WAVE = NINST / NWAVES;
  uint32_t voff[PER_WAVE];
  int first_row;

  __device__ __forceinline__ void init(int wave, int lane, uint32_t row_stride) {
    first_row = wave * PER_WAVE * RPI;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int row = first_row + i * RPI + lane / C;
      voff[i] = (uint32_t)row * row_stride + (uint32_t)(swz_chunk<ROWB>(row, lane % C) << 4);
    }
  }
  // Rows [0, valid_rows) of the tile start at `rows` (global) with stride `row_stride`.
  __device__ __forceinline__ void issue(const char* rows, int valid_rows, uint32_t row_stride,
                                        char* lds_tile) const {
    // The buffer descriptor type exists only for the GPU target; the host pass never runs
    // this body and must not see it (it would drop kernel launch stubs).
#if defined(__HIP_DEVICE_COMPILE__)
#if defined(ATTN_DEBUG_POISON_LDS)
    {
      const int lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
#pragma unroll
      for (int i = 0; i < PER_WAVE; ++i) poison16(lds_tile + (first_row + i * RPI) * ROWB + 16 * lane);
      poison_done();
    }
#endif
    const int v = valid_rows < 0 ? 0 : (valid_rows > ROWS ? ROWS : valid_rows);
    // The descriptor must live in scalar registers: every operand is workgroup-uniform.
    const uint64_t base = (uint64_t)rows;
    const uint64_t ubase = ((uint64_t)(uint32_t)uniform((int)(base >> 32)) << 32) |
                           (uint32_t)uniform((int)(uint32_t)base);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(ubase), (short)0, uniform((int)((uint32_t)v * row_stride)),
        0x00020000);
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rsrc, (__attribute__((address_space(3))) void*)(lds_tile + (first_row + i * RPI) * ROWB),
          16, voff[i], 0, 0, CPOL);
    }
#endif
  }
};

// ---------------------------------------------------------------------------------------
// V^T tiles for the bf16 PV contraction.
//
// The PV MFMA needs, per lane, 8 keys of one head-dim index: a column of the row-major V
// tile. Reading columns with the transposing LDS read moves only ~70 B/clk per CU on gfx950
// (measured), against ~220 B/clk for row-wise ds_read_b128, and every wave of a workgroup
// would repeat it. Instead the tile is transposed once per stage on its way into LDS:
// thread t loads 4 consecutive keys x 8 head-dim values (four 16-byte buffer loads, zeros
// past the sequence end), transposes that 4 x 8 block in registers with byte permutes, and
// writes eight 8-byte rows of V^T. The PV operands are then plain 16-byte reads.
//
// Layout: row d (head-dim index) holds the BN keys of the stage at a pitch of 2 BN + 16
// bytes (the 16-byte pad makes both the writes and the operand reads conflict-free on the
// 64-bank LDS). Within each group of 16 keys, key 8 j + 4 h + u sits at position
// 8 h + 4 j + u (bits 2 and 3 of the key index swapped), the order in which the P operand
// carries keys, so each lane's 8 keys of one MFMA step are contiguous.
// ---------------------------------------------------------------------------------------
template <int D, int BN>
struct VtStager {
  static constexpr int PITCH = 2 * BN + 16;
  static constexpr int TILE_BYTES = D * PITCH;
  static constexpr int GROUPS = BN / 4;                   // 4-key groups per stage
  static constexpr int ITEMS = GROUPS * (D / 8);          // (key group, head-dim chunk)
  static_assert(BN == 64 && ITEMS <= 256, "one item per thread of a 256-thread workgroup");
  uint32_t voff;   // global byte offset of key 4 m, chunk c, within the stage's rows
  int woff;        // LDS byte offset of row 8 c, position 4 m'
  bool active;
  i32x4 r[4];

  __device__ __forceinline__ void init(int tid, uint32_t row_stride) {
    const int m = tid % GROUPS, c = tid / GROUPS;
    active = tid < ITEMS;
    voff = (uint32_t)(4 * m) * row_stride + (uint32_t)(c * 16);
    const int mp = (m & ~3) | ((m & 1) << 1) | ((m >> 1) & 1);
    woff = 8 * c * PITCH + 8 * mp;
  }
  // Rows [0, valid_rows) of the stage start at `rows` (global) with stride `row_stride`.
  __device__ __forceinline__ void issue(const char* rows, int valid_rows, uint32_t row_stride) {
#if defined(__HIP_DEVICE_COMPILE__)
    const int v = valid_rows < 0 ? 0 : (valid_rows > BN ? BN : valid_rows);
    const uint64_t base = (uint64_t)rows;
    const uint64_t ubase = ((uint64_t)(uint32_t)uniform((int)(base >> 32)) << 32) |
                           (uint32_t)uniform((int)(uint32_t)base);
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        reinterpret_cast<void*>(ubase), (short)0, uniform((int)((uint32_t)v * row_stride)),
        0x00020000);
    if (ITEMS >= 256 || active) {  // branch-free when every thread stages (head_dim 128)
#pragma unroll
      for (int u = 0; u < 4; ++u)
        r[u] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                             rsrc, (int)(voff + (uint32_t)u * row_stride), 0, 0));
    }
#endif
  }
  // Race exposure: the sentinel into exactly the slots write() fills (see poison16).
  __device__ __forceinline__ void poison(char* lds_tile) const {
#if defined(ATTN_DEBUG_POISON_LDS)
    if (!active) return;
#pragma unroll
    for (int e = 0; e < 8; ++e) poison8(lds_tile + woff + e * PITCH);
    poison_done();
#endif
  }
  // Transpose the four loaded keys into eight V^T rows of 4 keys (8 bytes) each.
  __device__ __forceinline__ void write(char* lds_tile) const {
    if (!active) return;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      // head-dim 2e: low halves; 2e + 1: high halves (bytes 0,1 / 2,3 of each dword)
      const int lo01 = (int)__builtin_amdgcn_perm((uint32_t)r[1][e], (uint32_t)r[0][e], 0x05040100u);
      const int lo23 = (int)__builtin_amdgcn_perm((uint32_t)r[3][e], (uint32_t)r[2][e], 0x05040100u);
      const int hi01 = (int)__builtin_amdgcn_perm((uint32_t)r[1][e], (uint32_t)r[0][e], 0x07060302u);
      const int hi23 = (int)__builtin_amdgcn_perm((uint32_t)r[3][e], (uint32_t)r[2][e], 0x07060302u);
      *reinterpret_cast<i32x2*>(lds_tile + woff + (2 * e) * PITCH) = i32x2{lo01, lo23};
      *reinterpret_cast<i32x2*>(lds_tile + woff + (2 * e + 1) * PITCH) = i32x2{hi01, hi23};
    }
  }
};

// Wait for this thread's outstanding DMA / global loads (before the barrier that
// publishes an LDS stage).
__device__ __forceinline__ void wait_vmem() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Wait until at most N vector-memory operations of this thread are outstanding (loads
// complete in issue order): the N most recent loads may stay in flight.
template <int N>
__device__ __forceinline__ void wait_vmem_leave() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// ---------------------------------------------------------------------------------------
// Element-type specific contractions on swizzled tiles. Key k of a 32-key block sits in
// register r of lane half g = l / 32 with k = 8 * (r / 4) + 4 * g + (r % 4) (the
// accumulator layout above).
// ---------------------------------------------------------------------------------------
__device__ __forceinline__ int key_of_reg(int r, int g) { return 8 * (r >> 2) + 4 * g + (r & 3); }

template <typename T, int D>
struct Mma;

// bf16: v_mfma_f32_32x32x16_bf16 for both contractions; V^T operands via ds_read_b64_tr_b16.
template <int D>
struct Mma<__bf16, D> {
  static constexpr int ROWB = D * 2;
  static constexpr int QREGS = D / 16;
  static constexpr int NDB = D / 32;
  typedef bf16x8 QOperand;

  // Per-lane LDS byte offsets, fixed for the whole kernel.
  struct Offsets {
    int k[QREGS];    // K operand of step s: row l % 32, chunk 2 s + l / 32
    int v[NDB][2];   // V^T operand of head-dim block db, rows 8 j + 4 g + (l % 16) / 4
    int vt[NDB];     // V^T tile operand of head-dim block db: row 32 db + l % 32, +16 (l / 32)
  };
  __device__ static Offsets offsets(int lane) {
    Offsets o;
    const int i = lane & 31, g = lane >> 5;
#pragma unroll
    for (int s = 0; s < QREGS; ++s) o.k[s] = i * ROWB + (swz_chunk<ROWB>(i, 2 * s + g) << 4);
    const int a16 = lane & 15, hh = (lane >> 4) & 1;
    const int x = 4 * g + (a16 >> 2);  // row within an aligned group of 8
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int c = 4 * db + 2 * hh + ((a16 & 3) >> 1);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        o.v[db][j] = x * ROWB + (swz_chunk<ROWB>(8 * j + x, c) << 4) + 8 * (a16 & 1);
    }
#pragma unroll
    for (int db = 0; db < NDB; ++db)
      o.vt[db] = (32 * db + i) * VtStager<D, 64>::PITCH + 16 * g;
    return o;
  }

  // Q^T operand of S^T = K Q^T: lane (q = l % 32, g = l / 32) holds q[16 s + 8 g + 0..7].
  // `neg` flips the sign bit (exact) so a negative scale becomes a positive one.
  __device__ static void load_q(QOperand (&qr)[QREGS], const __bf16* qrow, bool valid, bool neg,
                                int lane) {
    const int g = lane >> 5;
#pragma unroll
    for (int s = 0; s < QREGS; ++s) {
      i32x4 x = valid ? *reinterpret_cast<const i32x4*>(qrow + 16 * s + 8 * g) : i32x4{0, 0, 0, 0};
      if (neg) x ^= i32x4{(int)0x80008000, (int)0x80008000, (int)0x80008000, (int)0x80008000};
      qr[s] = __builtin_bit_cast(bf16x8, x);
    }
  }

  // acc += K_block Q^T over the full head dimension; kl points at tile row 0 of the block
  // (a multiple of 8 rows into the tile).
  __device__ static void qk(f32x16& acc, const char* kl, const QOperand (&qr)[QREGS],
                            const Offsets& of, int lane) {
#pragma unroll
    for (int s = 0; s < QREGS; ++s) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(kl + of.k[s]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qr[s], acc, 0, 0, 0);
    }
  }

  // P^T operand of the two 16-key steps of a 32-key block, rounded to bf16.
  struct PPack {
    bf16x8 b[2];
    // Registers 2i, 2i+1 of the accumulator-layout P (round to nearest even).
    __device__ __forceinline__ void set_pair(int i, float e0, float e1) {
      typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
      typedef __attribute__((ext_vector_type(2))) float f32x2;
      const f32x2 x = {e0, e1};
      i32x4 w = __builtin_bit_cast(i32x4, b[i >> 2]);
      w[i & 3] = __builtin_bit_cast(int, __builtin_convertvector(x, bf16x2));
      b[i >> 2] = __builtin_bit_cast(bf16x8, w);
    }
  };
  // Rounds P to bf16 (round to nearest even, two values per instruction) and returns the
  // fp32 sum of the unrounded values: the saved LSE keeps fp32 accuracy.
  __device__ static float pack_p(const f32x16& p, PPack& pk) {
    typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
    typedef __attribute__((ext_vector_type(2))) float f32x2;
    float sum = p[0] + p[1];  // (a 0.0f start would cost an add: x + 0 is not x for -0)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      i32x4 w;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const f32x2 x = {p[8 * h + 2 * i], p[8 * h + 2 * i + 1]};
        w[i] = __builtin_bit_cast(int, __builtin_convertvector(x, bf16x2));
        if (h + i > 0) sum += x[0] + x[1];
      }
      pk.b[h] = __builtin_bit_cast(bf16x8, w);
    }
    return sum;
  }

  // o[db] += V_block^T P^T for the 32 keys of one block.
  // K-slot t = 4 j + u of step s carries key 16 s + 8 j + 4 g + u, which is register
  // 8 s + t of the accumulator-layout P, and is what the two transpose reads (rows +0 and
  // +8) return.
  __device__ static void pv(f32x16 (&o)[NDB], const PPack& pk, const char* vl, const Offsets& of,
                            int lane) {
    const bf16x8(&b)[2] = pk.b;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const char* p0 = vl + 16 * s * ROWB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + of.v[db][0]));
        const i16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p0 + 8 * ROWB + of.v[db][1]));
        const i32x4 cat = {__builtin_bit_cast(i32x2, lo)[0], __builtin_bit_cast(i32x2, lo)[1],
                           __builtin_bit_cast(i32x2, hi)[0], __builtin_bit_cast(i32x2, hi)[1]};
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, cat), b[s],
                                                        o[db], 0, 0, 0);
      }
    }
  }

  // Operand reads are issued PF MFMAs ahead of their use (one MFMA is shorter than an LDS
  // read's latency), and consecutive MFMAs write different accumulators. The scheduling
  // groups keep the compiler from clustering the reads back next to their MFMAs.
  static constexpr int PF = 4;

  // acc[kb] += K_kb Q^T for both 32-key blocks of a 64-key stage at `kt`.
  __device__ static void qk2(f32x16 (&acc)[2], const char* kt, const QOperand (&qr)[QREGS],
                             const Offsets& of) {
    constexpr int N = 2 * QREGS;  // MFMA i: block i & 1, head-dim step i >> 1
    bf16x8 a[N];
#pragma unroll
    for (int i = 0; i < PF; ++i)
      a[i] = *reinterpret_cast<const bf16x8*>(kt + (i & 1) * 32 * ROWB + of.k[i >> 1]);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (i + PF < N) {
        const int j = i + PF;
        a[j] = *reinterpret_cast<const bf16x8*>(kt + (j & 1) * 32 * ROWB + of.k[j >> 1]);
      }
      acc[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], qr[i >> 1], acc[i & 1], 0, 0, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
    for (int i = 0; i < N - PF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
  }

  // o[db] += V^T P^T over both 32-key blocks of a V^T tile (VtStager layout); MFMA i takes
  // block i / (2 NDB), step (i / NDB) & 1, head-dim block i % NDB.
  __device__ static void pv2(f32x16 (&o)[NDB], const PPack (&pk)[2], const char* vt_tile,
                             const Offsets& of) {
    constexpr int N = 4 * NDB;
    bf16x8 a[N];
#define ATTN_VT_OPERAND(i) \
  (*reinterpret_cast<const bf16x8*>(vt_tile + of.vt[(i) % NDB] + 64 * ((i) / (2 * NDB)) + 32 * (((i) / NDB) & 1)))
#pragma unroll
    for (int i = 0; i < PF; ++i) a[i] = ATTN_VT_OPERAND(i);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      if (i + PF < N) a[i + PF] = ATTN_VT_OPERAND(i + PF);
      o[i % NDB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          a[i], pk[i / (2 * NDB)].b[(i / NDB) & 1], o[i % NDB], 0, 0, 0);
    }
#undef ATTN_VT_OPERAND
    __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
    for (int i = 0; i < N - PF; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, PF, 0);
  }

  // o[db] += V_block^T P^T for the 32 keys of block kb of a V^T tile (VtStager layout):
  // step s reads positions 32 kb + 16 s + 8 (l / 32) + 0..7 of row 32 db + l % 32, which
  // hold keys 32 kb + 16 s + 8 j + 4 (l / 32) + u for slot t = 4 j + u: the keys the P
  // operand carries in slot t.
  __device__ static void pv_t(f32x16 (&o)[NDB], const PPack& pk, const char* vt_tile, int kb,
                              const Offsets& of) {
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(vt_tile + of.vt[db] + 64 * kb + 32 * s);
        o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pk.b[s], o[db], 0, 0, 0);
      }
    }
  }

  // Output element type conversion: four consecutive head-dim values -> 8 bytes.
  __device__ static void store4(__bf16* dst, float a, float b, float c, float d) {
    typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
    bf16x4 v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};
    *reinterpret_cast<bf16x4*>(dst) = v;
  }
};

// fp32: v_mfma_f32_32x32x2_f32 (exact products, fp32 accumulation).
template <int D>
struct Mma<float, D> {
  static constexpr int ROWB = D * 4;
  static constexpr int QREGS = D / 2;
  static constexpr int NDB = D / 32;
  typedef float QOperand;
  struct Offsets {};
  __device__ static Offsets offsets(int) { return Offsets{}; }

  __device__ static void load_q(QOperand (&qr)[QREGS], const float* qrow, bool valid, bool neg,
                                int lane) {
    const int g = lane >> 5;
#pragma unroll
    for (int s = 0; s < QREGS; ++s) {
      const float x = valid ? qrow[2 * s + g] : 0.0f;
      qr[s] = neg ? -x : x;
    }
  }

  // Element e of row r lives at r * ROWB + (swz(r, e / 4) << 4) + 4 (e % 4).
  __device__ static int at(int row, int e) {
    return row * ROWB + (swz_chunk<ROWB>(row, e >> 2) << 4) + 4 * (e & 3);
  }

  __device__ static void qk(f32x16& acc, const char* kl, const QOperand (&qr)[QREGS], const Offsets&,
                            int lane) {
    const int i = lane & 31, g = lane >> 5;
#pragma unroll
    for (int s = 0; s < QREGS; ++s) {
      const float a = *reinterpret_cast<const float*>(kl + at(i, 2 * s + g));
      acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a, qr[s], acc, 0, 0, 0);
    }
  }

  struct PPack {
    f32x16 p;
    __device__ __forceinline__ void set_pair(int i, float e0, float e1) {
      p[2 * i] = e0;
      p[2 * i + 1] = e1;
    }
  };
  __device__ static float pack_p(const f32x16& p, PPack& pk) {
    pk.p = p;
    float sum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) sum += p[r];
    return sum;
  }

  // Step r contracts the two keys held in register r by the two lane halves.
  __device__ static void pv(f32x16 (&o)[NDB], const PPack& pk, const char* vl, const Offsets&,
                            int lane) {
    const f32x16& p = pk.p;
    const int i = lane & 31, g = lane >> 5;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float a = *reinterpret_cast<const float*>(vl + at(key_of_reg(r, g), db * 32 + i));
        o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, p[r], o[db], 0, 0, 0);
      }
    }
  }

  __device__ static void store4(float* dst, float a, float b, float c, float d) {
    *reinterpret_cast<f32x4*>(dst) = f32x4{a, b, c, d};
  }
};

}  // namespace attn
