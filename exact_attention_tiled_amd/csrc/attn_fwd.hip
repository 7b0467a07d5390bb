// attn_fwd.hip - forward kernels: prefill, split-K decode + log-sum-exp combine, mask probe.
//
// Both forward kernels run the same per-wave step on a stage of keys staged in LDS:
//   S^T = K Q^T on MFMA (fp32 accumulate)  ->  exclusion of disallowed / out-of-range lanes
//   -> running max (per lane + one exchange with lane l^32)  ->  rescale of the denominator
//   and accumulator by exp2(m_old - m_new)  ->  P = exp2(scale*log2e*S - m_new)  ->
//   O^T += V^T P^T on MFMA,
// and divide by the denominator at the end ("Efficient Attention: Formal Correctness",
// "The FlashAttention Proof": online softmax recurrence; "Causal Mask and Ragged Sequence
// Layouts", sections 1-4: in-sequence positions, out-of-range lanes, alignment, zero rows).
#include <algorithm>
#include <type_traits>

#include "attn.h"
#include "attn_device.hpp"
#include "attn_internal.h"

namespace attn {

struct FwdParams {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_q;
  const int32_t* cu_k;
  int num_seqs, total_q, hq, hkv, group;
  float c2;   // |scale| * log2(e)
  int neg;    // scale < 0: sign folded into Q (exact)
  int mode, window;
  void* out;
  float* lse;
  // prefill: slot order (any lengths) or, for batches whose sequences all have the same
  // lengths, tiles of `uni_ntiles` per sequence enumerated heaviest first (uni_ntiles > 0)
  int nslots, nlogical;
  int uni_ntiles, npairs;
  int uni_lq, uni_lk;  // equal-length batch: every sequence's query / key length
  const int32_t* order;  // other batches: slots sorted by cost (prefill_order_kernel), -1 pads
  // split-K
  float* part_o;
  float* part_lse;
  int blocks_per_kvh, chunk, nsplit;
  // dropout (prefill kernel instantiated with DROP only)
  uint32_t seed_lo, seed_hi, drop_thr;
  float drop_scale;
  __bf16* out_res;  // bf16 (RES kernels only): rounding residual of O
};

// The exponent offset of a row moves only when a tile's maximum exceeds it by more than
// this many powers of two (or the row has seen nothing yet). Any offset gives the same
// O = acc / l and LSE = offset + log2 l; bounding every P by 2^8 keeps all terms finite, and
// most tiles then skip the accumulator rescale.
constexpr float RESCALE_THRESHOLD = 8.0f;

// One online-softmax step for NK key blocks of 32 keys held in accumulator layout.
// s[kb][r] is the raw (sign-folded) dot product of this lane's query with key
// kpos0 + 32 kb + key_of_reg(r, g); pk receives P (not yet normalised) as the PV operand.
// With need_mask the disallowed pairs are excluded first (mask_blocks).
// m_run is in log2 units of the scaled logits; l_run is this lane's partial denominator
// (the other half of the row lives in lane l ^ 32).
// With DROP the denominator still sums every weight, and the PV operand carries
// weight * keep / (1 - p) (the keep flags of DropoutSite for this lane's query). With RES
// (bf16, with or without DROP) that operand z is also split: pk gets bf16(z) and pkr
// bf16(z - bf16(z)), so that accumulating both against V gives the unrounded output to
// about 2^-16.
template <typename M, int NK, int D, bool DROP = false, bool RES = false>
__device__ __forceinline__ void softmax_step(f32x16 (&s)[NK], typename M::PPack (&pk)[NK],
                                             bool need_mask, int pq, int kpos0, const SeqGeom& g,
                                             int mode, int window, float c2, float& m_run,
                                             float& l_run, f32x16 (&o)[D / 32], int lane,
                                             const DropoutSite& drop = DropoutSite{},
                                             typename M::PPack* pkr = nullptr) {
  if (need_mask) mask_blocks<NK>(s, pq, kpos0, g, mode, window, lane);
  float mx = neg_inf();
#pragma unroll
  for (int kb = 0; kb < NK; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = max_halves(mx);
  const float mt = (mx == neg_inf()) ? neg_inf() : mx * c2;
  const bool grow = mt > m_run + RESCALE_THRESHOLD;
  if (__any(grow)) {
    const float m_new = grow ? mt : m_run;
    const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;  // 0 if nothing seen yet
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
    m_run = m_new;
  }
  const float base = (m_run == neg_inf()) ? 0.0f : m_run;
  if (need_mask) {
    // Excluded entries hold -inf; force their weight to exactly 0 (also when c2 == 0).
#pragma unroll
    for (int kb = 0; kb < NK; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float x = s[kb][r];
        const float e0 = fast_exp2(fmaf(x, c2, -base));
        s[kb][r] = (x == neg_inf()) ? 0.0f : e0;
      }
  } else {
#pragma unroll
    for (int kb = 0; kb < NK; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = fast_exp2(fmaf(s[kb][r], c2, -base));
  }
  if constexpr (DROP) {
    const int hg = lane >> 5;
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) {
      float sum = 0.0f;
#pragma unroll
      for (int r = 0; r < 16; ++r) sum += s[kb][r];
      l_run += sum;
      // registers 4a..4a+3 hold keys kpos0 + 32 kb + 8 a + 4 hg + 0..3
      uint32_t keep[4];
      dropout_keep_rows4(drop, pq, (kpos0 + 32 * kb + 4 * hg) >> 2, keep);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          s[kb][4 * a + b] = ((keep[a] >> b) & 1u) ? s[kb][4 * a + b] * drop.scale : 0.0f;
      if constexpr (RES) {
        f32x16 lo;
#pragma unroll
        for (int r = 0; r < 16; ++r) lo[r] = s[kb][r] - (float)(__bf16)s[kb][r];
        (void)M::pack_p(lo, pkr[kb]);
      }
      (void)M::pack_p(s[kb], pk[kb]);
    }
  } else {
#pragma unroll
    for (int kb = 0; kb < NK; ++kb) {
      if constexpr (RES) {
        f32x16 lo;
#pragma unroll
        for (int r = 0; r < 16; ++r) lo[r] = s[kb][r] - (float)(__bf16)s[kb][r];
        (void)M::pack_p(lo, pkr[kb]);
      }
      l_run += M::pack_p(s[kb], pk[kb]);
    }
  }
}

// The (query head, sequence, query tile) of this workgroup; false for padding blocks.
template <int BM>
__device__ __forceinline__ bool prefill_tile(const FwdParams& p, int& h, int& s, int& tile,
                                             SeqGeom& g) {
  if (p.uni_ntiles > 0) {
    // Equal-length batch. Block b takes tile rank b / npairs of (sequence, head) pair
    // b % npairs, so every tile of a given cost is dispatched before any cheaper one
    // (largest-first list scheduling), on every XCD alike. Heads are enumerated K/V head
    // fastest: with npairs a multiple of 8, the round-robin XCD assignment b % 8 then keeps
    // every query head of one GQA group, and all tiles of one (sequence, K/V head), on
    // the same XCD and its L2.
    const int b = blockIdx.x;
    const int rank = b / p.npairs, pair = b - rank * p.npairs;
    s = pair / p.hq;
    const int hp = pair - s * p.hq;
    h = (hp % p.hkv) * p.group + hp / p.hkv;
    // Every length equals its maximum, so cu_seqlens[s] = s * length: no loads needed.
    g.q_start = s * p.uni_lq;
    g.k_start = s * p.uni_lk;
    g.len_q = p.uni_lq;
    g.len_k = p.uni_lk;
    g.off = p.mode == MASK_BOTTOM_RIGHT ? p.uni_lk - p.uni_lq : 0;
    const int ntiles = (g.len_q + BM - 1) / BM;
    tile = p.uni_ntiles - 1 - rank;  // latest (heaviest under causal masks) tiles first
    return tile < ntiles;
  }
  int slot;
  if (p.order != nullptr) {
    // Block b takes sorted slot b / Hq for query head b % Hq, K/V head fastest: with Hq a
    // multiple of 8 the round-robin XCD assignment keeps each GQA group on one XCD.
    const int b = blockIdx.x;
    const int idx = b / p.hq, hp = b - idx * p.hq;
    slot = p.order[idx];
    if (slot < 0) return false;
    h = (hp % p.hkv) * p.group + hp / p.hkv;
  } else {
    const int w = xcd_logical_block(blockIdx.x, p.nlogical);
    if (w < 0) return false;
    h = w / p.nslots;
    slot = w - h * p.nslots;
  }
  s = seq_of_slot<BM>(p.cu_q, p.num_seqs, slot);
  g = load_geom(p.cu_q, p.cu_k, s, p.mode);
  const int ntiles = (g.len_q + BM - 1) / BM;
  const int j = slot - (g.q_start / BM + s);
  tile = ntiles - 1 - j;  // latest (heaviest under causal masks) tiles first
  return j < ntiles;
}

// Running state of one prefill wave (32 query rows) and its step over one 64-key stage.
// RES (bf16): the weights also go through V as their bf16 residuals.
template <typename T, int D, bool DROP = false, bool RES = false>
struct PrefillWave {
  typedef Mma<T, D> M;
  f32x16 o[D / 32];
  float m_run, l_run;

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    m_run = neg_inf();
    l_run = 0.0f;
  }

  // One stage of FWD_BN keys starting at key position k0: K tile at `kt` (row-major), V at
  // `vt` (V^T tile for bf16, row-major for fp32). The wave's rows are query positions
  // [wp0, wp1); this lane's query is pq.
  __device__ __forceinline__ void stage(const char* kt, const char* vt, int k0, int wp0, int wp1,
                                        int pq, const SeqGeom& g, const FwdParams& p,
                                        const typename M::QOperand (&qr)[M::QREGS],
                                        const typename M::Offsets& of, int lane,
                                        const DropoutSite& drop) {
    constexpr int ROWB = M::ROWB;
    const int cls = block_class(wp0, wp1, k0, k0 + FWD_BN, g, p.mode, p.window);
    if (cls == 0) return;
    f32x16 sacc[2];
    // The two waves sharing a SIMD alternate between MFMA and softmax phases: a wave
    // entering a contraction takes issue priority so the other wave's VALU work overlaps.
    __builtin_amdgcn_s_setprio(1);
    if constexpr (std::is_same<T, __bf16>::value) {
      sacc[0] = f32x16{};
      sacc[1] = f32x16{};
      M::qk2(sacc, kt, qr, of);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        sacc[kb] = f32x16{};
        M::qk(sacc[kb], kt + kb * 32 * ROWB, qr, of, lane);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    typename M::PPack pk[2], pkr[2];  // pkr: RES only
    softmax_step<M, 2, D, DROP, RES>(sacc, pk, cls == 1, pq, k0, g, p.mode, p.window, p.c2,
                                     m_run, l_run, o, lane, drop, pkr);
    __builtin_amdgcn_s_setprio(1);
    if constexpr (std::is_same<T, __bf16>::value) {
      M::pv2(o, pk, vt, of);
      if constexpr (RES) M::pv2(o, pkr, vt, of);
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) M::pv(o, pk[kb], vt + kb * 32 * ROWB, of, lane);
    }
    __builtin_amdgcn_s_setprio(0);
  }
};

// V staging of the prefill: bf16 transposes V into V^T tiles through registers (the
// loads of stage j+1 are in flight while stage j is computed, and written to LDS after
// it); fp32 copies row-major V tiles by DMA like K.
template <typename T, int D>
struct PrefillVStage {
  DmaStager<Mma<T, D>::ROWB, FWD_BN, 4> dma;
  static constexpr int TILE_BYTES = FWD_BN * Mma<T, D>::ROWB;
  __device__ __forceinline__ void init(int wave, int lane, int, uint32_t rstride) {
    dma.init(wave, lane, rstride);
  }
  __device__ __forceinline__ void issue(const char* rows, int valid, uint32_t rstride, char* tile) {
    dma.issue(rows, valid, rstride, tile);
  }
  __device__ __forceinline__ void commit(char*) const {}
};
template <int D>
struct PrefillVStage<__bf16, D> {
  VtStager<D, FWD_BN> vt;
  static constexpr int TILE_BYTES = VtStager<D, FWD_BN>::TILE_BYTES;
  __device__ __forceinline__ void init(int, int, int tid, uint32_t rstride) {
    vt.init(tid, rstride);
  }
  __device__ __forceinline__ void issue(const char* rows, int valid, uint32_t rstride, char* tile) {
    vt.poison(tile);  // (race-exposure builds only)
    vt.issue(rows, valid, rstride);
  }
  __device__ __forceinline__ void commit(char* tile) const { vt.write(tile); }
};

// ---------------------------------------------------------------------------------------
// Prefill: one workgroup = 4 waves = 128 query rows of one (sequence, query head); all
// waves share each 64-key K/V stage. Stages are DMA'd into two LDS buffers in turn: the
// load of stage j+1 is in flight while stage j is computed.
// ---------------------------------------------------------------------------------------
// With DROP the weights reaching V carry the dropout realisation (DropoutSite); this
// kernel is the forward of every dropout call. With RES (bf16) it also writes the output's
// rounding residual, with or without dropout.
template <typename T, int D, bool DROP = false, bool RES = false>
__global__ __launch_bounds__(256, 2) void fwd_prefill_kernel(FwdParams p) {
  static_assert(!RES || std::is_same<T, __bf16>::value, "residual: bf16 only");
  typedef Mma<T, D> M;
  constexpr int BM = FWD_BM, BN = FWD_BN, ROWB = M::ROWB;
  constexpr int KTILE = BN * ROWB, VTILE = PrefillVStage<T, D>::TILE_BYTES;
  static_assert(2 * (KTILE + VTILE) <= LDS_BYTES, "two K/V stages must fit in LDS");
  __shared__ __attribute__((aligned(1024))) char kbuf0[KTILE];
  __shared__ __attribute__((aligned(1024))) char kbuf1[KTILE];
  __shared__ __attribute__((aligned(1024))) char vbuf0[VTILE];
  __shared__ __attribute__((aligned(1024))) char vbuf1[VTILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  int h, s, tile;
  SeqGeom g;
  if (!prefill_tile<BM>(p, h, s, tile, g)) return;
  const int p0 = tile * BM, p1 = min(p0 + BM, g.len_q);
  const int kvh = h / p.group;

  // This wave's query rows and this lane's query.
  const int wp0 = p0 + 32 * wave, wp1 = min(wp0 + 32, p1);
  const int pq = wp0 + (lane & 31);
  const bool qvalid = pq < wp1;
  typename M::QOperand qr[M::QREGS];
  const T* qrow = static_cast<const T*>(p.q) + ((size_t)(g.q_start + pq) * p.hq + h) * D;
  M::load_q(qr, qrow, qvalid, p.neg != 0, lane);
  const typename M::Offsets of = M::offsets(lane);

  int klo, khi;
  visible_keys(p0, p1, g, p.mode, p.window, klo, khi);
  const int kstart = (klo / BN) * BN;
  const int nst = khi > klo ? (khi - kstart + BN - 1) / BN : 0;

  const uint32_t rstride = (uint32_t)(p.hkv * D * sizeof(T));
  const char* kb0 = static_cast<const char*>(p.k) + ((size_t)g.k_start * p.hkv + kvh) * D * sizeof(T);
  const char* vb0 = static_cast<const char*>(p.v) + ((size_t)g.k_start * p.hkv + kvh) * D * sizeof(T);
  DmaStager<ROWB, BN, 4> dma;
  dma.init(wave, lane, rstride);
  PrefillVStage<T, D> vst;
  vst.init(wave, lane, tid, rstride);

  PrefillWave<T, D, DROP, RES> st;
  st.init();
  DropoutSite drop{};
  if constexpr (DROP) drop = DropoutSite{p.seed_lo, p.seed_hi, p.drop_thr, p.drop_scale, s, h};

  // Stage j lives in buffer j % 2. The loads of stage j+1 are issued before stage j is
  // computed; the barrier after stage j publishes stage j+1 (the V^T transpose-write happens
  // once its loads have landed) and frees buffer j % 2 for stage j+2.
  if (nst > 0) {
    dma.issue(kb0 + (size_t)kstart * rstride, g.len_k - kstart, rstride, kbuf0);
    vst.issue(vb0 + (size_t)kstart * rstride, g.len_k - kstart, rstride, vbuf0);
  }
  wait_vmem();
  if (nst > 0) vst.commit(vbuf0);
  __syncthreads();
  for (int it = 0; it < nst; it += 2) {
    const int k0 = kstart + it * BN;
    if (it + 1 < nst) {
      dma.issue(kb0 + (size_t)(k0 + BN) * rstride, g.len_k - k0 - BN, rstride, kbuf1);
      vst.issue(vb0 + (size_t)(k0 + BN) * rstride, g.len_k - k0 - BN, rstride, vbuf1);
    }
    st.stage(kbuf0, vbuf0, k0, wp0, wp1, pq, g, p, qr, of, lane, drop);
    wait_vmem();
    if (it + 1 < nst) vst.commit(vbuf1);
    __syncthreads();
    if (it + 1 < nst) {
      if (it + 2 < nst) {
        dma.issue(kb0 + (size_t)(k0 + 2 * BN) * rstride, g.len_k - k0 - 2 * BN, rstride, kbuf0);
        vst.issue(vb0 + (size_t)(k0 + 2 * BN) * rstride, g.len_k - k0 - 2 * BN, rstride, vbuf0);
      }
      st.stage(kbuf1, vbuf1, k0 + BN, wp0, wp1, pq, g, p, qr, of, lane, drop);
      wait_vmem();
      if (it + 2 < nst) vst.commit(vbuf0);
      __syncthreads();
    }
  }
  f32x16 (&o)[D / 32] = st.o;
  const float m_run = st.m_run, l_run = st.l_run;

  // Epilogue: O = acc / l (exactly +0.0 for rows that saw no allowed key), natural-log LSE.
  const float lt = sum_halves(l_run);
  const bool nonempty = lt > 0.0f;
  const float inv = nonempty ? 1.0f / lt : 0.0f;
  if (qvalid) {
    T* orow = static_cast<T*>(p.out) + ((size_t)(g.q_start + pq) * p.hq + h) * D;
    const int hg = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = db * 32 + 8 * a + 4 * hg;
        M::store4(orow + d, nonempty ? o[db][4 * a] * inv : 0.0f,
                  nonempty ? o[db][4 * a + 1] * inv : 0.0f, nonempty ? o[db][4 * a + 2] * inv : 0.0f,
                  nonempty ? o[db][4 * a + 3] * inv : 0.0f);
      }
    if constexpr (RES) {
      // The residual x - bf16(x) of every stored element (bf16, |r| <= half an ulp of the
      // output), so that the backward can form D = rowsum(dO * O) from the unrounded O.
      __bf16* rrow = p.out_res + ((size_t)(g.q_start + pq) * p.hq + h) * D;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          float x[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float y = nonempty ? o[db][4 * a + e] * inv : 0.0f;
            x[e] = y - (float)(__bf16)y;
          }
          M::store4(rrow + db * 32 + 8 * a + 4 * hg, x[0], x[1], x[2], x[3]);
        }
    }
    if (hg == 0)
      p.lse[(size_t)h * p.total_q + g.q_start + pq] =
          nonempty ? (m_run + fast_log2(lt)) * LN2 : neg_inf();
  }
}

// ---------------------------------------------------------------------------------------
// bf16 prefill, software-pipelined within each wave. Iteration j issues the MFMAs of
// S_j = K_j Q^T and, while the matrix core works through them, evaluates the exponentials
// of stage j-1 on the vector ALUs (scheduling groups interleave the two instruction
// streams); it then accumulates O += V_{j-1}^T P_{j-1}^T. K_{j+1} is DMA'd during
// iteration j; V_j is loaded into registers at the start of iteration j and written as a
// V^T tile at its end, ready for iteration j+1. One barrier per iteration.
// ---------------------------------------------------------------------------------------

// First half of the online-softmax step for the two 32-key blocks of a stage: exclusion of
// disallowed pairs (-inf), row maximum, lazy rescale of l and O. Returns the exponent
// offset the stage's weights are taken against.
template <int D>
__device__ __forceinline__ float stage_max(f32x16 (&s)[2], bool need_mask, int pq, int kpos0,
                                           const SeqGeom& g, int mode, int window, float c2,
                                           float& m_run, float& l_run, f32x16 (&o)[D / 32],
                                           int lane) {
  if (need_mask) mask_blocks<2>(s, pq, kpos0, g, mode, window, lane);
  float mx = neg_inf();
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = max_halves(mx);
  const float mt = (mx == neg_inf()) ? neg_inf() : mx * c2;
  const bool grow = mt > m_run + RESCALE_THRESHOLD;
  if (__any(grow)) {
    const float m_new = grow ? mt : m_run;
    const float alpha = grow ? fast_exp2(m_run - m_new) : 1.0f;  // 0 if nothing seen yet
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
    m_run = m_new;
  }
  return (m_run == neg_inf()) ? 0.0f : m_run;
}

// Second half: P = exp2(c2 S - base) as the bf16 PV operand; returns the fp32 sum of the
// unrounded weights. Excluded pairs hold -inf and give exactly 0 (c2 > 0).
template <int D>
__device__ __forceinline__ float stage_exp(f32x16 (&s)[2], typename Mma<__bf16, D>::PPack (&pk)[2],
                                           float c2, float base) {
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) s[kb][r] = fast_exp2(fmaf(s[kb][r], c2, -base));
  return Mma<__bf16, D>::pack_p(s[0], pk[0]) + Mma<__bf16, D>::pack_p(s[1], pk[1]);
}

// S_new = K_tile Q^T for both 32-key blocks, with the exponentials of the previous stage
// (s_old -> pk) interleaved: per MFMA one operand read (PF ahead) and ~7 VALU instructions.
// `issue` requests the next stage's K and V; its 8 buffer loads are spread over the first
// 8 MFMAs. Issuing them in a burst before the contraction stalled the wave for ~400 cycles
// per stage while the CU's memory pipeline accepted them (measured with per-phase cycle
// stamps); behind the MFMAs that wait overlaps matrix work.
template <int D, typename Issue>
__device__ __forceinline__ float qk_with_exp(const Issue& issue, f32x16 (&sn)[2], const char* kt,
                                             const bf16x8 (&qr)[D / 16],
                                             const typename Mma<__bf16, D>::Offsets& of,
                                             f32x16 (&so)[2],
                                             typename Mma<__bf16, D>::PPack (&pk)[2], float c2,
                                             float base) {
  typedef Mma<__bf16, D> M;
  constexpr int ROWB = M::ROWB, N = 2 * M::QREGS, PF = M::PF;
  bf16x8 a[N];
#pragma unroll
  for (int i = 0; i < PF; ++i)
    a[i] = *reinterpret_cast<const bf16x8*>(kt + (i & 1) * 32 * ROWB + of.k[i >> 1]);
  issue();
  sn[0] = f32x16{};
  sn[1] = f32x16{};
#pragma unroll
  for (int i = 0; i < N; ++i) {
    if (i + PF < N) {
      const int j = i + PF;
      a[j] = *reinterpret_cast<const bf16x8*>(kt + (j & 1) * 32 * ROWB + of.k[j >> 1]);
    }
    sn[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], qr[i >> 1], sn[i & 1], 0, 0, 0);
  }
  const float sum = stage_exp<D>(so, pk, c2, base);
  constexpr int NV = (112 + N - 1) / N;  // fma + exp per weight, bf16 packs, fp32 sums
  __builtin_amdgcn_sched_group_barrier(0x100, PF, 0);
#pragma unroll
  for (int i = 0; i < N; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    if (i < 8) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
    if (i + PF < N) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
  }
  return sum;
}

// Loop-invariant operands and geometry of one pipelined prefill wave.
template <int D>
struct PipeCtx {
  typedef Mma<__bf16, D> M;
  const FwdParams& p;
  const SeqGeom& g;
  const bf16x8 (&qr)[D / 16];
  const typename M::Offsets& of;
  DmaStager<2 * D, FWD_BN, 4>& dma;
  VtStager<D, FWD_BN>& vst;
  const char* kg;
  const char* vg;
  uint32_t rstride;
  int nst, kstart, wp0, wp1, pq, lane;
};

// Running state: O accumulator, exponent offset, partial denominator.
template <int D>
struct PipeRun {
  f32x16 o[D / 32];
  float m_run, l_run;
  bool mask_prev;  // the stage whose weights are pending needs per-lane masking
};

// Steady iteration j (0 < j < nst): stage j's K in kbuf[B] (B = j % 2), stage j-1's scores
// in `so`, its V^T in vbuf[B ^ 1]; stage j's scores go to `sn`.
template <int D, int B>
__device__ __forceinline__ void prefill_steady(const PipeCtx<D>& c, PipeRun<D>& r, int j,
                                               f32x16 (&sn)[2], f32x16 (&so)[2],
                                               char* const (&kbuf)[2], char* const (&vbuf)[2]) {
  typedef Mma<__bf16, D> M;
  constexpr int BN = FWD_BN;
  const int kcur = c.kstart + j * BN;
  // K_{j+1} (DMA) and V_j (registers). In the last iteration the K request covers no row
  // (a select, not a branch: a branch would split the block and stop the scheduler from
  // spreading the requests over the MFMAs): the descriptor's range check turns it into zero
  // writes to a buffer nothing reads, without fetching keys that no row of the tile sees.
  auto issue = [&]() {
    c.dma.issue(c.kg + (size_t)(kcur + BN) * c.rstride, j + 1 < c.nst ? c.g.len_k - kcur - BN : 0,
                c.rstride, kbuf[B ^ 1]);
    c.vst.poison(vbuf[B]);  // (race-exposure builds only) V^T_j lands there at the end
    c.vst.issue(c.vg + (size_t)kcur * c.rstride, c.g.len_k - kcur, c.rstride);
  };
  const float base = stage_max<D>(so, r.mask_prev, c.pq, kcur - BN, c.g, c.p.mode, c.p.window,
                                  c.p.c2, r.m_run, r.l_run, r.o, c.lane);
  typename M::PPack pk[2];
  // The two workgroups sharing a CU alternate: a wave in its contractions takes issue
  // priority, so the co-resident wave's softmax and staging fill the MFMA shadow.
  __builtin_amdgcn_s_setprio(1);
  r.l_run += qk_with_exp<D>(issue, sn, kbuf[B], c.qr, c.of, so, pk, c.p.c2, base);
  M::pv2(r.o, pk, vbuf[B ^ 1], c.of);
  __builtin_amdgcn_s_setprio(0);
  r.mask_prev = block_class(c.wp0, c.wp1, kcur, kcur + BN, c.g, c.p.mode, c.p.window) != 2;
  wait_vmem();
  c.vst.write(vbuf[B]);
  __syncthreads();
}

// Last step: weights and PV of stage nst - 1 (scores in `so`, V^T in vbuf[B]).
template <int D, int B>
__device__ __forceinline__ void prefill_tail(const PipeCtx<D>& c, PipeRun<D>& r,
                                             f32x16 (&so)[2], char* const (&vbuf)[2]) {
  typedef Mma<__bf16, D> M;
  const int klast = c.kstart + (c.nst - 1) * FWD_BN;
  const float base = stage_max<D>(so, r.mask_prev, c.pq, klast, c.g, c.p.mode, c.p.window,
                                  c.p.c2, r.m_run, r.l_run, r.o, c.lane);
  typename M::PPack pk[2];
  r.l_run += stage_exp<D>(so, pk, c.p.c2, base);
  M::pv2(r.o, pk, vbuf[B], c.of);
}

template <int D>
__global__ __launch_bounds__(256, 2) void fwd_prefill_bf16_kernel(FwdParams p) {
  typedef Mma<__bf16, D> M;
  typedef VtStager<D, FWD_BN> VS;
  constexpr int BM = FWD_BM, BN = FWD_BN, ROWB = M::ROWB, KTILE = BN * ROWB;
  static_assert(2 * (KTILE + VS::TILE_BYTES) <= LDS_BYTES / 2, "two workgroups per CU");
  __shared__ __attribute__((aligned(1024))) char kbuf0[KTILE];
  __shared__ __attribute__((aligned(1024))) char kbuf1[KTILE];
  __shared__ __attribute__((aligned(1024))) char vbuf0[VS::TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char vbuf1[VS::TILE_BYTES];
  char* const kbuf[2] = {kbuf0, kbuf1};
  char* const vbuf[2] = {vbuf0, vbuf1};

  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  int h, s, tile;
  SeqGeom g;
  if (!prefill_tile<BM>(p, h, s, tile, g)) return;
  const int p0 = tile * BM, p1 = min(p0 + BM, g.len_q);
  const int kvh = h / p.group;
  const int wp0 = p0 + 32 * wave, wp1 = min(wp0 + 32, p1);
  const int pq = wp0 + (lane & 31);
  const bool qvalid = pq < wp1;
  bf16x8 qr[M::QREGS];
  const typename M::Offsets of = M::offsets(lane);

  int kstart, nst;
  stage_range(p0, p1, g, p.mode, p.window, BN, kstart, nst);

  const uint32_t rstride = (uint32_t)(p.hkv * D * 2);
  const char* kg = static_cast<const char*>(p.k) + ((size_t)g.k_start * p.hkv + kvh) * D * 2;
  const char* vg = static_cast<const char*>(p.v) + ((size_t)g.k_start * p.hkv + kvh) * D * 2;
  DmaStager<ROWB, BN, 4> dma;
  dma.init(wave, lane, rstride);
  VS vst;
  vst.init(tid, rstride);

  PipeRun<D> r;
#pragma unroll
  for (int db = 0; db < D / 32; ++db) r.o[db] = f32x16{};
  r.m_run = neg_inf();
  r.l_run = 0.0f;
  r.mask_prev = true;
  const PipeCtx<D> c{p, g, qr, of, dma, vst, kg, vg, rstride, nst, kstart, wp0, wp1, pq, lane};
  f32x16 sa[2], sb[2];  // scores of even / odd stages

  if (nst > 0) {
    // The tile's Q arrives by DMA as two 64-row halves in the V^T buffers (free until stage
    // 0's V^T is written): whole 256-byte rows per request instead of the 32-byte pieces of
    // the operand layout. Then K_0, V_0 and K_1: everything is requested before the first
    // wait, so the tile's start costs one memory round trip, not three.
    {
      const uint32_t qstride = (uint32_t)(p.hq * D * 2);
      const char* qg = static_cast<const char*>(p.q) + ((size_t)(g.q_start + p0) * p.hq + h) * D * 2;
      DmaStager<ROWB, 64, 4> qdma;
      qdma.init(wave, lane, qstride);
      qdma.issue(qg, p1 - p0, qstride, vbuf0);
      qdma.issue(qg + (size_t)64 * qstride, p1 - p0 - 64, qstride, vbuf1);
    }
    dma.issue(kg + (size_t)kstart * rstride, g.len_k - kstart, rstride, kbuf0);
    vst.issue(vg + (size_t)kstart * rstride, g.len_k - kstart, rstride);
    if (nst > 1) {
      dma.issue(kg + (size_t)(kstart + BN) * rstride, g.len_k - kstart - BN, rstride, kbuf1);
      // Wait for Q and K_0 only (this wave issued 4 V loads if it stages V, then K_1).
      if (vst.active)
        wait_vmem_leave<DmaStager<ROWB, BN, 4>::PER_WAVE + 4>();
      else
        wait_vmem_leave<DmaStager<ROWB, BN, 4>::PER_WAVE>();
    } else {
      wait_vmem();
    }
    __syncthreads();
    {
      // This wave's 32 Q rows as QK^T operands (rows past the tile end arrived as zeros);
      // the operand layout is the K tile's, so the K offsets apply.
      const char* qt = (wave < 2 ? vbuf0 : vbuf1) + (wave & 1) * 32 * ROWB;
      const int flip = p.neg != 0 ? (int)0x80008000 : 0;  // negative scale: flip Q's sign
#pragma unroll
      for (int st = 0; st < M::QREGS; ++st) {
        i32x4 x = *reinterpret_cast<const i32x4*>(qt + of.k[st]);
        x ^= i32x4{flip, flip, flip, flip};
        qr[st] = __builtin_bit_cast(bf16x8, x);
      }
    }
    // Stage 0: scores only. Under a window its keys can lie before every row of a lower
    // wave: that wave takes -inf scores instead of the contraction (its weights are then
    // exact zeros, as the per-lane test would make them).
    const int cls0 = block_class(wp0, wp1, kstart, kstart + BN, g, p.mode, p.window);
    if (cls0 == 0) {
#pragma unroll
      for (int r2 = 0; r2 < 16; ++r2) {
        sa[0][r2] = neg_inf();
        sa[1][r2] = neg_inf();
      }
    } else {
      sa[0] = f32x16{};
      sa[1] = f32x16{};
      M::qk2(sa, kbuf0, qr, of);
    }
    r.mask_prev = cls0 == 1;
    wait_vmem();
    __syncthreads();  // every wave has its Q operands: vbuf0 takes V^T_0
    vst.poison(vbuf0);
    vst.write(vbuf0);
    __syncthreads();
    int j = 1;
    for (; j + 1 < nst; j += 2) {
      prefill_steady<D, 1>(c, r, j, sb, sa, kbuf, vbuf);
      prefill_steady<D, 0>(c, r, j + 1, sa, sb, kbuf, vbuf);
    }
    // Under a causal mask the last stage holds keys that the upper rows of the tile never
    // see: a wave none of whose rows sees any of them leaves out that stage's weights and
    // PV contraction (a uniform branch; they would add exact zeros).
    const int klast = kstart + (nst - 1) * BN;
    const bool skip_last =
        nst > 1 && block_class(wp0, wp1, klast, klast + BN, g, p.mode, p.window) == 0;
    if (j < nst) {
      prefill_steady<D, 1>(c, r, j, sb, sa, kbuf, vbuf);
      if (!skip_last) prefill_tail<D, 1>(c, r, sb, vbuf);
    } else {
      if (!skip_last) prefill_tail<D, 0>(c, r, sa, vbuf);
    }
  }

  // Epilogue: O = acc / l (exactly +0.0 for rows that saw no allowed key), natural-log LSE.
  const float lt = sum_halves(r.l_run);
  const bool nonempty = lt > 0.0f;
  const float inv = nonempty ? 1.0f / lt : 0.0f;
  // O goes through LDS so that every store instruction writes whole 256-byte rows: in the
  // accumulator layout a lane holds 8-byte pieces of one row, and storing those directly
  // costs 32 partial-row writes per instruction. The K buffers are free here (the last K
  // read preceded the last barrier; other waves may still read V^T), 8 KB per wave.
  {
    char* ot = (wave < 2 ? kbuf[0] : kbuf[1]) + (wave & 1) * 32 * ROWB;
    const int i = lane & 31, hg = lane >> 5;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        // head-dim 32 db + 8 a + 4 hg + 0..3: 8 bytes in 16-byte chunk 4 db + a of row i
        M::store4(reinterpret_cast<__bf16*>(ot + i * ROWB + (swz_chunk<ROWB>(i, 4 * db + a) << 4) + 8 * hg),
                  nonempty ? r.o[db][4 * a] * inv : 0.0f, nonempty ? r.o[db][4 * a + 1] * inv : 0.0f,
                  nonempty ? r.o[db][4 * a + 2] * inv : 0.0f, nonempty ? r.o[db][4 * a + 3] * inv : 0.0f);
      }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    constexpr int CPR = ROWB / 16, RPI = 64 / CPR;  // 16-byte chunks per row, rows per instruction
    const int c = lane % CPR;
    const size_t rstep = (size_t)p.hq * D;
    __bf16* obase = static_cast<__bf16*>(p.out) + ((size_t)(g.q_start + wp0) * p.hq + h) * D;
#pragma unroll
    for (int k = 0; k < 32 / RPI; ++k) {
      const int row = k * RPI + lane / CPR;
      const i32x4 x = *reinterpret_cast<const i32x4*>(ot + row * ROWB + (swz_chunk<ROWB>(row, c) << 4));
      // Nontemporal: O is not read again by this call, and its lines would otherwise
      // displace K/V lines that other tiles still read from L2.
      if (wp0 + row < wp1)
        __builtin_nontemporal_store(x, reinterpret_cast<i32x4*>(obase + row * rstep + 8 * c));
    }
  }
  if (qvalid && lane < 32)
    p.lse[(size_t)h * p.total_q + g.q_start + pq] =
        nonempty ? (r.m_run + fast_log2(lt)) * LN2 : neg_inf();
}

// Running state of one split-K wave: one block of 32 query rows over KBW consecutive
// 32-key blocks of each stage.
template <typename T, int D, int KBW>
struct SplitkWave {
  typedef Mma<T, D> M;
  f32x16 o[D / 32];
  float m_run, l_run;

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int db = 0; db < D / 32; ++db) o[db] = f32x16{};
    m_run = neg_inf();
    l_run = 0.0f;
  }

  // Keys [kw0, kw0 + 32 KBW) of a stage, staged at kt / vt (row 0 = key kw0); rows
  // [rlo, rhi) of the group's G * len_q (position, head) rows; only keys in [klo, khi)
  // (this workgroup's chunk) count.
  __device__ __forceinline__ void stage(const char* kt, const char* vt, int kw0, int klo, int khi,
                                        int rlo, int rhi, int pq, const SeqGeom& g,
                                        const FwdParams& p,
                                        const typename M::QOperand (&qr)[M::QREGS],
                                        const typename M::Offsets& of, int lane) {
    constexpr int ROWB = M::ROWB;
    bool clip;
    const int cls = splitk_stage_class<KBW>(kw0, klo, khi, rlo, rhi, g, p.group, p.mode,
                                            p.window, clip);
    if (cls == 0) return;
    f32x16 sacc[KBW];
#pragma unroll
    for (int i = 0; i < KBW; ++i) {
      sacc[i] = f32x16{};
      M::qk(sacc[i], kt + 32 * i * ROWB, qr, of, lane);
    }
    const bool need_mask = splitk_stage_clip<KBW>(sacc, cls, clip, kw0, klo, khi, lane);
    typename M::PPack pk[KBW];
    softmax_step<M, KBW, D>(sacc, pk, need_mask, pq, kw0, g, p.mode, p.window, p.c2, m_run,
                            l_run, o, lane);
#pragma unroll
    for (int i = 0; i < KBW; ++i) M::pv(o, pk[i], vt + 32 * i * ROWB, of, lane);
  }
};

// ---------------------------------------------------------------------------------------
// Split-K decode: one workgroup = one (sequence, K/V head, key chunk). Its rows are the
// G * len_q (query head, query position) pairs of the group, so every K/V byte is read
// once for the whole group. With NRB row blocks of 32, wave w owns row block w % NRB and
// KBW = NRB consecutive 32-key blocks of every 128-key stage (the waves sharing a row
// block split the stage's keys); each wave keeps its own running state, the waves of a row
// block merge their states at the end, and the chunk writes one partial (O_e normalised,
// LSE_e), e = chunk. The combine kernel merges the partials of each row.
// ---------------------------------------------------------------------------------------
template <typename T, int D, int NRB>
__global__ __launch_bounds__(256, 1) void fwd_splitk_kernel(FwdParams p) {
  typedef Mma<T, D> M;
  constexpr int BN = SPLITK_STAGE, ROWB = M::ROWB;
  constexpr int TILE = BN * ROWB;
  constexpr int KW = 4 / NRB, KBW = NRB;  // waves per row block, key blocks per wave
  static_assert(2 * 2 * TILE <= LDS_BYTES, "two K/V stages must fit in LDS");
  __shared__ __attribute__((aligned(1024))) char buf0[2 * TILE];
  __shared__ __attribute__((aligned(1024))) char buf1[2 * TILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int b = blockIdx.x;
  const int sigma = b % p.blocks_per_kvh;
  const int kvh = (b / p.blocks_per_kvh) % p.hkv;
  const int s = b / (p.blocks_per_kvh * p.hkv);
  const SeqGeom g = load_geom(p.cu_q, p.cu_k, s, p.mode);
  const int G = p.group;
  const int R = G * g.len_q;
  if (R == 0) return;

  // This wave's rows: r = position * G + head-in-group, r in [rlo, rhi).
  const int rb = wave % NRB, kwi = wave / NRB;
  const int rlo = rb * 32, rhi = min(R, rlo + 32);
  const int r = rlo + (lane & 31);
  const bool rvalid = r < R;
  const int pq = rvalid ? r / G : 0;
  typename M::QOperand qr[M::QREGS];
  {
    const int h = kvh * G + (rvalid ? r % G : 0);
    const T* qrow = static_cast<const T*>(p.q) + ((size_t)(g.q_start + pq) * p.hq + h) * D;
    M::load_q(qr, qrow, rvalid, p.neg != 0, lane);
  }
  const typename M::Offsets of = M::offsets(lane);

  int vlo, vhi;
  visible_keys(0, g.len_q, g, p.mode, p.window, vlo, vhi);
  const int klo = max(vlo, sigma * p.chunk);
  const int khi = min(vhi, sigma * p.chunk + p.chunk);
  const int kstart = (klo / BN) * BN;
  const int nst = khi > klo ? (khi - kstart + BN - 1) / BN : 0;

  const uint32_t rstride = (uint32_t)(p.hkv * D * sizeof(T));
  const char* kb0 = static_cast<const char*>(p.k) + ((size_t)g.k_start * p.hkv + kvh) * D * sizeof(T);
  const char* vb0 = static_cast<const char*>(p.v) + ((size_t)g.k_start * p.hkv + kvh) * D * sizeof(T);
  DmaStager<ROWB, BN, 4, CPOL_NT> dma;  // every K/V byte is read once per call
  dma.init(wave, lane, rstride);

  // This wave's key blocks start at block kwi * KBW of each stage.
  const int woff = 32 * kwi * KBW;
  SplitkWave<T, D, KBW> st;
  st.init();
  if (nst > 0) {
    dma.issue(kb0 + (size_t)kstart * rstride, g.len_k - kstart, rstride, buf0);
    dma.issue(vb0 + (size_t)kstart * rstride, g.len_k - kstart, rstride, buf0 + TILE);
  }
  wait_vmem();
  __syncthreads();
  for (int it = 0; it < nst; it += 2) {
    const int k0 = kstart + it * BN;
    if (it + 1 < nst) {
      dma.issue(kb0 + (size_t)(k0 + BN) * rstride, g.len_k - k0 - BN, rstride, buf1);
      dma.issue(vb0 + (size_t)(k0 + BN) * rstride, g.len_k - k0 - BN, rstride, buf1 + TILE);
    }
    st.stage(buf0 + woff * ROWB, buf0 + TILE + woff * ROWB, k0 + woff, klo, khi, rlo, rhi, pq, g,
             p, qr, of, lane);
    wait_vmem();
    __syncthreads();
    if (it + 1 < nst) {
      if (it + 2 < nst) {
        dma.issue(kb0 + (size_t)(k0 + 2 * BN) * rstride, g.len_k - k0 - 2 * BN, rstride, buf0);
        dma.issue(vb0 + (size_t)(k0 + 2 * BN) * rstride, g.len_k - k0 - 2 * BN, rstride, buf0 + TILE);
      }
      st.stage(buf1 + woff * ROWB, buf1 + TILE + woff * ROWB, k0 + BN + woff, klo, khi, rlo, rhi,
               pq, g, p, qr, of, lane);
      wait_vmem();
      __syncthreads();
    }
  }

  // The KW waves of a row block hold partial softmax states (O unnormalised, offset m in
  // log2 units, denominator l) over disjoint keys of the chunk. They are merged here through
  // LDS (the stage buffers are free after the last barrier), so the chunk writes ONE partial
  // per row: M = max m_w, l = sum l_w 2^(m_w - M), O = sum O_w 2^(m_w - M). Waves that saw
  // no key (m_w = -inf) weigh 0.
  constexpr int NO = D / 32 * 16;  // O values per lane
  float lt = sum_halves(st.l_run);
  float mt = st.m_run;
  if constexpr (KW > 1) {
    float* red = reinterpret_cast<float*>(buf0);  // per (row block, wave > 0): O, m, l
    constexpr int SLOT = (NO + 2) * 64;
    static_assert(NRB * (KW - 1) * SLOT * 4 <= 2 * TILE, "merge area must fit one stage buffer");
    if (kwi > 0) {
      float* sl = red + (rb * (KW - 1) + kwi - 1) * SLOT;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) sl[(db * 16 + i) * 64 + lane] = st.o[db][i];
      sl[NO * 64 + lane] = mt;
      sl[(NO + 1) * 64 + lane] = lt;
    }
    __syncthreads();
    if (kwi == 0) {
      float mw[KW], lw[KW];
      mw[0] = mt;
      lw[0] = lt;
#pragma unroll
      for (int w = 1; w < KW; ++w) {
        const float* sl = red + (rb * (KW - 1) + w - 1) * SLOT;
        mw[w] = sl[NO * 64 + lane];
        lw[w] = sl[(NO + 1) * 64 + lane];
      }
      float mm = mw[0];
#pragma unroll
      for (int w = 1; w < KW; ++w) mm = fmaxf(mm, mw[w]);
      float sc[KW];
      lt = 0.0f;
#pragma unroll
      for (int w = 0; w < KW; ++w) {
        sc[w] = mw[w] == neg_inf() ? 0.0f : fast_exp2(mw[w] - mm);
        lt += lw[w] * sc[w];
      }
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float acc = st.o[db][i] * sc[0];
#pragma unroll
          for (int w = 1; w < KW; ++w)
            acc += red[(rb * (KW - 1) + w - 1) * SLOT + (db * 16 + i) * 64 + lane] * sc[w];
          st.o[db][i] = acc;
        }
      mt = mm;
    }
  }

  // The row block's partial for this chunk: normalised O_e (fp32) and LSE_e; empty -> O_e = 0,
  // LSE_e = -inf.
  const int e = sigma;
  const int hg = lane >> 5;
  const bool nonempty = lt > 0.0f;
  const float inv = nonempty ? 1.0f / lt : 0.0f;
  if (kwi == 0 && rvalid) {
    const int t = g.q_start + pq;
    const int h = kvh * G + r % G;
    float* dst = p.part_o + (((size_t)e * p.total_q + t) * p.hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = db * 32 + 8 * a + 4 * hg;
        *reinterpret_cast<f32x4*>(dst + d) =
            f32x4{nonempty ? st.o[db][4 * a] * inv : 0.0f, nonempty ? st.o[db][4 * a + 1] * inv : 0.0f,
                  nonempty ? st.o[db][4 * a + 2] * inv : 0.0f, nonempty ? st.o[db][4 * a + 3] * inv : 0.0f};
      }
    if (hg == 0)
      p.part_lse[((size_t)e * p.hq + h) * p.total_q + t] =
          nonempty ? (mt + fast_log2(lt)) * LN2 : neg_inf();
  }
}

// Log-sum-exp combine of split partials: LSE = log sum_e exp(LSE_e);
// O = sum_e exp(LSE_e - LSE) O_e; every partial empty -> O = +0.0, LSE = -inf.
// One wave per (query token, query head).
template <typename T, int D>
__global__ __launch_bounds__(256) void splitk_combine_kernel(const float* __restrict__ part_o,
                                                             const float* __restrict__ part_lse,
                                                             int nsplit, int total_q, int hq,
                                                             T* __restrict__ out,
                                                             float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= total_q * hq) return;
  const int t = item / hq, h = item - (item / hq) * hq;
  constexpr int PER = D / 64;
  float m = neg_inf();
  for (int e = 0; e < nsplit; ++e) m = fmaxf(m, part_lse[((size_t)e * hq + h) * total_q + t]);
  float acc[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) acc[i] = 0.0f;
  float sum = 0.0f;
  if (m != neg_inf()) {
    for (int e = 0; e < nsplit; ++e) {
      const float le = part_lse[((size_t)e * hq + h) * total_q + t];
      if (le == neg_inf()) continue;
      const float wgt = fast_exp2((le - m) * LOG2E);
      sum += wgt;
      const float* src = part_o + (((size_t)e * total_q + t) * hq + h) * D;
#pragma unroll
      for (int i = 0; i < PER; ++i) acc[i] += wgt * src[lane * PER + i];
    }
  }
  const bool nonempty = sum > 0.0f;
  const float inv = nonempty ? 1.0f / sum : 0.0f;
  T* dst = out + ((size_t)t * hq + h) * D;
#pragma unroll
  for (int i = 0; i < PER; ++i) dst[lane * PER + i] = (T)(nonempty ? acc[i] * inv : 0.0f);
  if (lane == 0) lse[(size_t)h * total_q + t] = nonempty ? m + logf(sum) : neg_inf();
}

// ---------------------------------------------------------------------------------------
// Mask probes. Each replays one kernel's exclusion decisions for a query token on a zero
// score tile, with the functions that kernel calls in the same composition: its stage
// range, the per-wave block class of every stage, and the per-lane tests (mask_blocks; the
// split-K chunk clip). One 64-lane wave per query token t; its lanes hold t's query with
// the two lane halves' key registers, as in the kernels. Every key whose score is still
// finite (or whose block is wholly allowed) enters the softmax: bits[(t - q0) * nk +
// (u - k0)] = 1 for it (the array is zeroed first).
// ---------------------------------------------------------------------------------------
__global__ void probe_zero_kernel(uint8_t* bits, long n) {
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (long)gridDim.x * blockDim.x)
    bits[i] = 0;
}

// Marks the keys of NK 32-key blocks at kpos0 (accumulator layout) whose score is finite.
template <int NK>
__device__ __forceinline__ void probe_mark(const f32x16 (&s)[NK], int kpos0, const SeqGeom& g,
                                           int k0, int nk, uint8_t* row, int lane) {
  const int hg = lane >> 5;
#pragma unroll
  for (int kb = 0; kb < NK; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int u = g.k_start + kpos0 + 32 * kb + key_of_reg(r, hg);
      if (s[kb][r] != neg_inf() && u >= k0 && u < k0 + nk) row[u - k0] = 1;
    }
}

// Prefill. PIPELINED: the bf16 kernel (every visited stage runs mask_blocks unless the
// block class says every pair is allowed); otherwise the generic kernel (fp32, dropout:
// class 0 stages are skipped, class 1 stages masked).
template <bool PIPELINED>
__global__ void mask_probe_prefill_kernel(const int32_t* cu_q, const int32_t* cu_k, int num_seqs,
                                          int mode, int window, int q0, int nq, int k0, int nk,
                                          uint8_t* bits) {
  const int t = q0 + blockIdx.x, lane = threadIdx.x;
  const int s = seq_of_token(cu_q, num_seqs, t);
  const SeqGeom g = load_geom(cu_q, cu_k, s, mode);
  const int pq = t - g.q_start;
  const int p0 = (pq / FWD_BM) * FWD_BM, p1 = min(p0 + FWD_BM, g.len_q);
  const int wp0 = p0 + ((pq - p0) / 32) * 32, wp1 = min(wp0 + 32, p1);
  int kstart, nst;
  stage_range(p0, p1, g, mode, window, FWD_BN, kstart, nst);
  uint8_t* row = bits + (size_t)blockIdx.x * nk;
  for (int st = 0; st < nst; ++st) {
    const int kp = kstart + st * FWD_BN;
    const int cls = block_class(wp0, wp1, kp, kp + FWD_BN, g, mode, window);
    if (!PIPELINED && cls == 0) continue;
    f32x16 sc[2] = {f32x16{}, f32x16{}};
    if (PIPELINED ? cls != 2 : cls == 1) mask_blocks<2>(sc, pq, kp, g, mode, window, lane);
    probe_mark<2>(sc, kp, g, k0, nk, row, lane);
  }
}

// Split-K decode with nsb key chunks of `chunk` keys per (sequence, K/V head), for query
// head h: the rows of the group are (position, head-in-group) pairs, row pq * G + h % G;
// its row block is owned by the waves w with w % NRB equal to it, each of which takes KBW
// = NRB consecutive 32-key blocks of every 128-key stage.
template <int NRB>
__global__ void mask_probe_splitk_kernel(const int32_t* cu_q, const int32_t* cu_k, int num_seqs,
                                         int mode, int window, int group, int h, int nsb,
                                         int chunk, int q0, int nq, int k0, int nk,
                                         uint8_t* bits) {
  constexpr int KW = 4 / NRB, KBW = NRB, BN = SPLITK_STAGE;
  const int t = q0 + blockIdx.x, lane = threadIdx.x;
  const int s = seq_of_token(cu_q, num_seqs, t);
  const SeqGeom g = load_geom(cu_q, cu_k, s, mode);
  const int pq = t - g.q_start;
  const int R = group * g.len_q;
  const int r = pq * group + h % group;
  const int rlo = (r / 32) * 32, rhi = min(R, rlo + 32);
  int vlo, vhi;
  visible_keys(0, g.len_q, g, mode, window, vlo, vhi);
  uint8_t* row = bits + (size_t)blockIdx.x * nk;
  for (int sigma = 0; sigma < nsb; ++sigma) {
    const int klo = max(vlo, sigma * chunk), khi = min(vhi, sigma * chunk + chunk);
    const int kstart = (klo / BN) * BN;
    const int nst = khi > klo ? (khi - kstart + BN - 1) / BN : 0;
    for (int st = 0; st < nst; ++st)
      for (int kwi = 0; kwi < KW; ++kwi) {
        const int kw0 = kstart + st * BN + 32 * kwi * KBW;
        bool clip;
        const int cls = splitk_stage_class<KBW>(kw0, klo, khi, rlo, rhi, g, group, mode, window,
                                                clip);
        if (cls == 0) continue;
        f32x16 sc[KBW];
#pragma unroll
        for (int i = 0; i < KBW; ++i) sc[i] = f32x16{};
        if (splitk_stage_clip<KBW>(sc, cls, clip, kw0, klo, khi, lane))
          mask_blocks<KBW>(sc, pq, kw0, g, mode, window, lane);
        probe_mark<KBW>(sc, kw0, g, k0, nk, row, lane);
      }
  }
}

// The dropout realisation as the kernels compute it: one wave per 32 x 32 block of (query,
// key) positions, both positions 32-aligned as in every kernel's blocks. Row form (forward,
// dQ): lane l holds query qb + l % 32, register group a the keys kb + 8 a + 4 (l / 32) + 0..3.
// Column form (dK, dV): lane l holds key kb + l % 32, group a the queries
// qb + 8 a + 4 (l / 32) + 0..3. keep[i * nk + j] bit 0 is the row form's flag of (q0 + i,
// k0 + j), bit 1 the column form's.
__global__ void __launch_bounds__(64) dropout_probe_kernel(DropoutSite d, int q0, int nq,
                                                           int k0, int nk, uint8_t* keep) {
  __shared__ uint8_t tile[32][33];
  const int lane = threadIdx.x, hg = lane >> 5, li = lane & 31;
  const int qb = (q0 & ~31) + 32 * (int)blockIdx.y, kb = (k0 & ~31) + 32 * (int)blockIdx.x;
  uint32_t rows[4], cols[4];
  dropout_keep_rows4(d, qb + li, (kb + 4 * hg) >> 2, rows);
  dropout_keep_cols4(d, (qb + 4 * hg) >> 2, kb + li, cols);
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) tile[li][8 * a + 4 * hg + b] = (uint8_t)((rows[a] >> b) & 1u);
  __syncthreads();
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      tile[8 * a + 4 * hg + v][li] |= (uint8_t)(((cols[a] >> v) & 1u) << 1);
  __syncthreads();
  for (int e = lane; e < 32 * 32; e += 64) {
    const int i = qb + (e >> 5) - q0, j = kb + (e & 31) - k0;
    if (i >= 0 && i < nq && j >= 0 && j < nk) keep[(long)i * nk + j] = tile[e >> 5][e & 31];
  }
}

// ---------------------------------------------------------------------------------------
// Tile order of a prefill over sequences of different lengths. Every (sequence, query
// tile) slot gets its cost - the number of 64-key stages its rows visit - and the slots
// are sorted by cost, most first, with a counting sort in one workgroup (buckets beyond
// ORDER_BUCKETS - 1 stages share the last one). The prefill then dispatches the heaviest
// tiles first over all sequences (largest-first list scheduling), instead of in sequence
// order, where the long tiles of the last sequences ran last and left a tail. Padding
// slots (a sequence has fewer tiles than its slot range) are dropped; entries past the
// valid count are -1. Ties are written in atomic order: tiles are independent, so the
// order changes no result.
// ---------------------------------------------------------------------------------------
constexpr int ORDER_BUCKETS = 4096;
constexpr int ORDER_THREADS = 1024;

// (per lane: every lane of the sorting workgroup has its own slot)
template <int BM>
__device__ __forceinline__ int slot_cost(const int32_t* cu_q, const int32_t* cu_k, int num_seqs,
                                         int mode, int window, int slot) {
  int lo = 0, hi = num_seqs - 1;  // sequence of the slot: largest s with cu_q[s] / BM + s <= slot
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] / BM + mid <= slot) lo = mid; else hi = mid - 1;
  }
  const int s = lo;
  const SeqGeom g = load_geom_lane(cu_q, cu_k, s, mode);
  const int ntiles = (g.len_q + BM - 1) / BM;
  const int j = slot - (g.q_start / BM + s);
  if (j >= ntiles) return -1;
  const int tile = ntiles - 1 - j;
  const int p0 = tile * BM, p1 = min(p0 + BM, g.len_q);
  int kstart, nst;
  stage_range(p0, p1, g, mode, window, FWD_BN, kstart, nst);
  return min(nst, ORDER_BUCKETS - 1);
}

template <int BM>
__global__ __launch_bounds__(ORDER_THREADS) void prefill_order_kernel(
    const int32_t* cu_q, const int32_t* cu_k, int num_seqs, int nslots, int mode, int window,
    int32_t* order) {
  constexpr int PER = ORDER_BUCKETS / ORDER_THREADS;
  __shared__ int hist[ORDER_BUCKETS];
  __shared__ int part[ORDER_THREADS];
  const int tid = threadIdx.x;
  for (int b = tid; b < ORDER_BUCKETS; b += ORDER_THREADS) hist[b] = 0;
  __syncthreads();
  for (int slot = tid; slot < nslots; slot += ORDER_THREADS) {
    const int c = slot_cost<BM>(cu_q, cu_k, num_seqs, mode, window, slot);
    if (c >= 0) atomicAdd(&hist[c], 1);
  }
  __syncthreads();
  // First position of each cost: the number of slots that cost more. Thread t owns the
  // PER buckets ORDER_BUCKETS - 1 - PER t - i (descending); a scan over the threads' sums.
  int local[PER], sum = 0;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    local[i] = hist[ORDER_BUCKETS - 1 - PER * tid - i];
    sum += local[i];
  }
  part[tid] = sum;
  __syncthreads();
  for (int off = 1; off < ORDER_THREADS; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - sum;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    hist[ORDER_BUCKETS - 1 - PER * tid - i] = run;
    run += local[i];
  }
  const int count = part[ORDER_THREADS - 1];
  __syncthreads();
  for (int slot = tid; slot < nslots; slot += ORDER_THREADS) {
    const int c = slot_cost<BM>(cu_q, cu_k, num_seqs, mode, window, slot);
    if (c >= 0) order[atomicAdd(&hist[c], 1)] = slot;
  }
  for (int i = count + tid; i < nslots; i += ORDER_THREADS) order[i] = -1;
}

// ---------------------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------------------
static FwdParams make_params(const FwdArgs& a) {
  FwdParams p{};
  p.q = a.q;
  p.k = a.k;
  p.v = a.v;
  p.cu_q = a.cu_q;
  p.cu_k = a.cu_k;
  p.num_seqs = a.num_seqs;
  p.total_q = a.total_q;
  p.hq = a.hq;
  p.hkv = a.hkv;
  p.group = a.hq / a.hkv;
  const double c2 = (a.scale < 0 ? -(double)a.scale : (double)a.scale) * 1.4426950408889634;
  // A zero scale runs as the smallest normal float: every allowed weight is then exactly 1
  // (|s| * 2^-126 rounds away inside exp2), and -inf * c2 stays -inf for excluded pairs.
  p.c2 = std::max((float)c2, 1.17549435e-38f);
  p.neg = a.scale < 0;
  p.mode = a.mode;
  p.window = a.window;
  p.out = a.out;
  p.lse = a.lse;
  return p;
}

// Every sequence has max_q queries and max_k keys exactly when the totals say so (each
// length is at most its maximum).
bool equal_lengths(const FwdArgs& a) {
  return a.max_q > 0 && (long)a.total_q == (long)a.num_seqs * a.max_q &&
         (long)a.total_k == (long)a.num_seqs * a.max_k;
}

int fwd_prefill_grid(const FwdArgs& a) {
  const long ntiles = (a.max_q + FWD_BM - 1) / FWD_BM;
  if (equal_lengths(a)) return (int)(ntiles * a.num_seqs * a.hq);
  const long nslots = (long)a.total_q / FWD_BM + a.num_seqs;
  return (int)(nslots * a.hq);
}

size_t fwd_prefill_workspace_bytes(const FwdArgs& a) {
  if (equal_lengths(a)) return 0;
  const size_t nslots = (size_t)a.total_q / FWD_BM + a.num_seqs;
  return ((nslots * sizeof(int32_t) + 255) / 256) * 256;
}

template <typename T, int D>
static hipError_t prefill_typed(const FwdArgs& a, void* ws, hipStream_t st) {
  FwdParams p = make_params(a);
  p.nslots = a.total_q / FWD_BM + a.num_seqs;
  p.nlogical = p.nslots * a.hq;
  if (equal_lengths(a)) {
    p.uni_ntiles = (a.max_q + FWD_BM - 1) / FWD_BM;
    p.npairs = a.num_seqs * a.hq;
    p.uni_lq = a.max_q;
    p.uni_lk = a.max_k;
  } else {
    p.order = static_cast<const int32_t*>(ws);
    hipLaunchKernelGGL((prefill_order_kernel<FWD_BM>), dim3(1), dim3(ORDER_THREADS), 0, st,
                       a.cu_q, a.cu_k, a.num_seqs, p.nslots, a.mode, a.window,
                       static_cast<int32_t*>(ws));
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int grid = fwd_prefill_grid(a);
  if (a.drop_thr > 0) {
    p.seed_lo = (uint32_t)a.seed;
    p.seed_hi = (uint32_t)(a.seed >> 32);
    p.drop_thr = a.drop_thr;
    p.drop_scale = a.drop_scale;
    p.out_res = static_cast<__bf16*>(a.out_res);
    if constexpr (std::is_same<T, __bf16>::value) {
      if (p.out_res != nullptr) {
        hipLaunchKernelGGL((fwd_prefill_kernel<T, D, true, true>), dim3(grid), dim3(256), 0, st,
                           p);
        return hipGetLastError();
      }
    }
    hipLaunchKernelGGL((fwd_prefill_kernel<T, D, true>), dim3(grid), dim3(256), 0, st, p);
  } else if constexpr (std::is_same<T, __bf16>::value) {
    if (a.out_res != nullptr) {
      // No dropout, but the caller wants the output's rounding residual (an exact D for the
      // backward): the unpipelined kernel with the split PV operand.
      p.out_res = static_cast<__bf16*>(a.out_res);
      hipLaunchKernelGGL((fwd_prefill_kernel<T, D, false, true>), dim3(grid), dim3(256), 0, st,
                         p);
      return hipGetLastError();
    }
    hipLaunchKernelGGL((fwd_prefill_bf16_kernel<D>), dim3(grid), dim3(256), 0, st, p);
  } else {
    hipLaunchKernelGGL((fwd_prefill_kernel<T, D>), dim3(grid), dim3(256), 0, st, p);
  }
  return hipGetLastError();
}

hipError_t launch_fwd_prefill(const FwdArgs& a, void* ws, hipStream_t st) {
  if (a.dtype == 0)
    return a.d == 64 ? prefill_typed<__bf16, 64>(a, ws, st) : prefill_typed<__bf16, 128>(a, ws, st);
  return a.d == 64 ? prefill_typed<float, 64>(a, ws, st) : prefill_typed<float, 128>(a, ws, st);
}

int splitk_partials_per_chunk(int) { return 1; }

size_t splitk_workspace_bytes(int nsplit_eff, int total_q, int hq, int d) {
  const size_t o = (size_t)nsplit_eff * total_q * hq * d * sizeof(float);
  const size_t l = (size_t)nsplit_eff * hq * total_q * sizeof(float);
  return ((o + 255) / 256) * 256 + ((l + 255) / 256) * 256;
}

template <typename T, int D>
static hipError_t splitk_typed(const FwdArgs& a, int nsb, int chunk, void* ws, hipStream_t st) {
  FwdParams p = make_params(a);
  p.blocks_per_kvh = nsb;
  p.chunk = chunk;
  const int rows = (a.hq / a.hkv) * a.max_q;
  p.nsplit = nsb * splitk_partials_per_chunk(rows);
  const size_t obytes = (size_t)p.nsplit * a.total_q * a.hq * D * sizeof(float);
  p.part_o = static_cast<float*>(ws);
  p.part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + ((obytes + 255) / 256) * 256);
  const int grid = a.num_seqs * a.hkv * nsb;
  if (rows <= 32)
    hipLaunchKernelGGL((fwd_splitk_kernel<T, D, 1>), dim3(grid), dim3(256), 0, st, p);
  else
    hipLaunchKernelGGL((fwd_splitk_kernel<T, D, 2>), dim3(grid), dim3(256), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int items = a.total_q * a.hq;
  hipLaunchKernelGGL((splitk_combine_kernel<T, D>), dim3((items + 3) / 4), dim3(256), 0, st,
                     p.part_o, p.part_lse, p.nsplit, a.total_q, a.hq, static_cast<T*>(a.out), a.lse);
  return hipGetLastError();
}

hipError_t launch_fwd_splitk(const FwdArgs& a, int nsb, int chunk, void* ws, hipStream_t st) {
  if (a.dtype == 0)
    return a.d == 64 ? splitk_typed<__bf16, 64>(a, nsb, chunk, ws, st)
                     : splitk_typed<__bf16, 128>(a, nsb, chunk, ws, st);
  // fp32 with head_dim 128: two 128-key stages do not fit in LDS; the planner never
  // selects split-K for it.
  return a.d == 64 ? splitk_typed<float, 64>(a, nsb, chunk, ws, st) : hipErrorNotSupported;
}

hipError_t launch_probe_zero(uint8_t* bits, long n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const long blocks = std::min<long>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(probe_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, bits, n);
  return hipGetLastError();
}

hipError_t launch_mask_probe_fwd(const ProbeArgs& a, uint8_t* bits, hipStream_t st) {
  hipError_t e = launch_probe_zero(bits, (long)a.nq * a.nk, st);
  if (e != hipSuccess || a.nq == 0) return e;
  const dim3 grid(a.nq), block(64);
  if (a.unit == 0)
    hipLaunchKernelGGL((mask_probe_prefill_kernel<true>), grid, block, 0, st, a.cu_q, a.cu_k,
                       a.num_seqs, a.mode, a.window, a.q0, a.nq, a.k0, a.nk, bits);
  else if (a.unit == 1)
    hipLaunchKernelGGL((mask_probe_prefill_kernel<false>), grid, block, 0, st, a.cu_q, a.cu_k,
                       a.num_seqs, a.mode, a.window, a.q0, a.nq, a.k0, a.nk, bits);
  else if (a.nrb == 1)
    hipLaunchKernelGGL((mask_probe_splitk_kernel<1>), grid, block, 0, st, a.cu_q, a.cu_k,
                       a.num_seqs, a.mode, a.window, a.group, a.head, a.nsb, a.chunk, a.q0, a.nq,
                       a.k0, a.nk, bits);
  else
    hipLaunchKernelGGL((mask_probe_splitk_kernel<2>), grid, block, 0, st, a.cu_q, a.cu_k,
                       a.num_seqs, a.mode, a.window, a.group, a.head, a.nsb, a.chunk, a.q0, a.nq,
                       a.k0, a.nk, bits);
  return hipGetLastError();
}

// cu_seqlens checks. Thread i looks at sequences i, i + 256, ...; the bits meet in LDS and
// thread 0 writes the word (always, so the caller's word needs no clearing).
__global__ __launch_bounds__(256) void check_seqlens_kernel(const int32_t* cu_q,
                                                            const int32_t* cu_k, int num_seqs,
                                                            int total_q, int total_k, int max_q,
                                                            int max_k, int32_t* word) {
  __shared__ int bits;
  const int tid = threadIdx.x;
  if (tid == 0) bits = 0;
  __syncthreads();
  int b = 0;
  for (int s = tid; s < num_seqs; s += blockDim.x) {
    const long lq = (long)cu_q[s + 1] - cu_q[s], lk = (long)cu_k[s + 1] - cu_k[s];
    if (lq < 0) b |= ATTN_SEQLENS_Q_DECREASING;
    if (lq > max_q) b |= ATTN_SEQLENS_Q_ABOVE_MAX;
    if (lk < 0) b |= ATTN_SEQLENS_K_DECREASING;
    if (lk > max_k) b |= ATTN_SEQLENS_K_ABOVE_MAX;
  }
  if (tid == 0) {
    if (cu_q[0] != 0) b |= ATTN_SEQLENS_Q_START;
    if (cu_q[num_seqs] != total_q) b |= ATTN_SEQLENS_Q_END;
    if (cu_k[0] != 0) b |= ATTN_SEQLENS_K_START;
    if (cu_k[num_seqs] != total_k) b |= ATTN_SEQLENS_K_END;
  }
  if (b != 0) atomicOr(&bits, b);
  __syncthreads();
  if (tid == 0) *word = bits;
}

hipError_t launch_check_seqlens(const int32_t* cu_q, const int32_t* cu_k, int num_seqs,
                                int total_q, int total_k, int max_q, int max_k, int32_t* word,
                                hipStream_t st) {
  hipLaunchKernelGGL(check_seqlens_kernel, dim3(1), dim3(256), 0, st, cu_q, cu_k, num_seqs,
                     total_q, total_k, max_q, max_k, word);
  return hipGetLastError();
}

hipError_t launch_dropout_probe(uint64_t seed, uint32_t thr, int s, int h, int q0, int nq, int k0,
                                int nk, uint8_t* keep, hipStream_t st) {
  const DropoutSite d{(uint32_t)seed, (uint32_t)(seed >> 32), thr, 1.0f, s, h};
  const dim3 grid((unsigned)(((k0 + nk + 31) >> 5) - (k0 >> 5)),
                  (unsigned)(((q0 + nq + 31) >> 5) - (q0 >> 5)));
  hipLaunchKernelGGL(dropout_probe_kernel, grid, dim3(64), 0, st, d, q0, nq, k0, nk, keep);
  return hipGetLastError();
}

}  // namespace attn
