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
  // prefill
  int nslots, nlogical;
  // split-K
  float* part_o;
  float* part_lse;
  int blocks_per_kvh, chunk, nsplit;
};

// The exponent offset of a row moves only when a tile's maximum exceeds it by more than
// this many powers of two (or the row has seen nothing yet). Any offset gives the same
// O = acc / l and LSE = offset + log2 l; bounding every P by 2^8 keeps all terms finite, and
// most tiles then skip the accumulator rescale.
constexpr float RESCALE_THRESHOLD = 8.0f;

// One online-softmax step for NK key blocks of 32 keys held in accumulator layout.
// s[kb][r] is the raw (sign-folded) dot product of this lane's query with key
// kpos0 + 32 kb + key_of_reg(r, g); pk receives P (not yet normalised) as the PV operand.
// m_run is in log2 units of the scaled logits; l_run is this lane's partial denominator
// (the other half of the row lives in lane l ^ 32).
template <typename M, int NK, int D>
__device__ __forceinline__ void softmax_step(f32x16 (&s)[NK], typename M::PPack (&pk)[NK],
                                             bool need_mask, int pq, int kpos0, const SeqGeom& g,
                                             int mode, int window, float c2, float& m_run,
                                             float& l_run, f32x16 (&o)[D / 32], int lane) {
  const int hg = lane >> 5;
  if (need_mask) {
#pragma unroll
    for (int kb = 0; kb < NK; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const bool ok = pair_allowed(pq, kpos0 + 32 * kb + key_of_reg(r, hg), g, mode, window);
        s[kb][r] = ok ? s[kb][r] : neg_inf();
      }
  }
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
#pragma unroll
  for (int kb = 0; kb < NK; ++kb) l_run += M::pack_p(s[kb], pk[kb]);
}

// Running state of one prefill wave (32 query rows) and its step over one 64-key stage.
template <typename T, int D>
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

  // One stage of FWD_BN keys starting at key position k0, staged at `buf` (K tile, then
  // V tile). The wave's rows are query positions [wp0, wp1); this lane's query is pq.
  __device__ __forceinline__ void stage(const char* buf, int k0, int wp0, int wp1, int pq,
                                        const SeqGeom& g, const FwdParams& p,
                                        const typename M::QOperand (&qr)[M::QREGS],
                                        const typename M::Offsets& of, int lane) {
    constexpr int ROWB = M::ROWB, TILE = FWD_BN * ROWB;
    const int cls = block_class(wp0, wp1, k0, k0 + FWD_BN, g, p.mode, p.window);
    if (cls == 0) return;
    f32x16 sacc[2];
    // The two waves sharing a SIMD alternate between MFMA and softmax phases: a wave
    // entering a contraction takes issue priority so the other wave's VALU work overlaps.
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      sacc[kb] = f32x16{};
      M::qk(sacc[kb], buf + kb * 32 * ROWB, qr, of, lane);
    }
    __builtin_amdgcn_s_setprio(0);
    typename M::PPack pk[2];
    softmax_step<M, 2, D>(sacc, pk, cls == 1, pq, k0, g, p.mode, p.window, p.c2, m_run, l_run, o,
                          lane);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) M::pv(o, pk[kb], buf + TILE + kb * 32 * ROWB, of, lane);
    __builtin_amdgcn_s_setprio(0);
  }
};

// ---------------------------------------------------------------------------------------
// Prefill: one workgroup = 4 waves = 128 query rows of one (sequence, query head); all
// waves share each 64-key K/V stage. Stages are DMA'd into two LDS buffers in turn: the
// load of stage j+1 is in flight while stage j is computed.
// ---------------------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256, 2) void fwd_prefill_kernel(FwdParams p) {
  typedef Mma<T, D> M;
  constexpr int BM = FWD_BM, BN = FWD_BN, ROWB = M::ROWB;
  constexpr int TILE = BN * ROWB;
  static_assert(2 * 2 * TILE <= LDS_BYTES, "two K/V stages must fit in LDS");
  __shared__ __attribute__((aligned(1024))) char buf0[2 * TILE];  // K tile, then V tile
  __shared__ __attribute__((aligned(1024))) char buf1[2 * TILE];

  const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
  const int w = xcd_logical_block(blockIdx.x, p.nlogical);
  if (w < 0) return;
  const int h = w / p.nslots, slot = w - h * p.nslots;
  const int s = seq_of_slot<BM>(p.cu_q, p.num_seqs, slot);
  const SeqGeom g = load_geom(p.cu_q, p.cu_k, s, p.mode);
  const int ntiles = (g.len_q + BM - 1) / BM;
  const int j = slot - (g.q_start / BM + s);
  if (j >= ntiles) return;
  const int tile = ntiles - 1 - j;  // latest (heaviest under causal masks) tiles first
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

  PrefillWave<T, D> st;
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
    st.stage(buf0, k0, wp0, wp1, pq, g, p, qr, of, lane);
    wait_vmem();
    __syncthreads();
    if (it + 1 < nst) {
      if (it + 2 < nst) {
        dma.issue(kb0 + (size_t)(k0 + 2 * BN) * rstride, g.len_k - k0 - 2 * BN, rstride, buf0);
        dma.issue(vb0 + (size_t)(k0 + 2 * BN) * rstride, g.len_k - k0 - 2 * BN, rstride, buf0 + TILE);
      }
      st.stage(buf1, k0 + BN, wp0, wp1, pq, g, p, qr, of, lane);
      wait_vmem();
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
    if (hg == 0)
      p.lse[(size_t)h * p.total_q + g.q_start + pq] =
          nonempty ? (m_run + fast_log2(lt)) * LN2 : neg_inf();
  }
}

// Running state of one split-K wave (NRB blocks of 32 query rows) and its step over its
// 32-key block of one 128-key stage.
template <typename T, int D, int NRB>
struct SplitkWave {
  typedef Mma<T, D> M;
  f32x16 o[NRB][D / 32];
  float m_run[NRB], l_run[NRB];

  __device__ __forceinline__ void init() {
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[rb][db] = f32x16{};
      m_run[rb] = neg_inf();
      l_run[rb] = 0.0f;
    }
  }

  __device__ __forceinline__ void stage(const char* buf, int k0, int klo, int khi, int R, int wave,
                                        const int (&pq)[NRB], const SeqGeom& g,
                                        const FwdParams& p,
                                        const typename M::QOperand (&qr)[NRB][M::QREGS],
                                        const typename M::Offsets& of, int lane) {
    constexpr int ROWB = M::ROWB, TILE = SPLITK_STAGE * ROWB;
    const int G = p.group;
    const int kw = k0 + 32 * wave;  // this wave's key block
    // A key outside this block's chunk belongs to a neighbouring chunk's partial.
    const int cw0 = max(kw, klo), cw1 = min(kw + 32, khi);
#pragma unroll
    for (int rb = 0; rb < NRB; ++rb) {
      const int rlo = rb * 32, rhi = min(R, rb * 32 + 32);
      const int cls = (rhi <= rlo || cw1 <= cw0)
                          ? 0
                          : block_class(rlo / G, (rhi - 1) / G + 1, kw, kw + 32, g, p.mode, p.window);
      if (cls == 0) continue;
      const bool clip = cw0 != kw || cw1 != kw + 32;
      f32x16 sacc[1];
      sacc[0] = f32x16{};
      M::qk(sacc[0], buf + 32 * wave * ROWB, qr[rb], of, lane);
      if (clip) {
        const int hg = lane >> 5;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kk = kw + key_of_reg(r, hg);
          sacc[0][r] = ((kk >= cw0) & (kk < cw1)) ? sacc[0][r] : neg_inf();
        }
      }
      typename M::PPack pk[1];
      softmax_step<M, 1, D>(sacc, pk, cls == 1 || clip, pq[rb], kw, g, p.mode, p.window, p.c2,
                            m_run[rb], l_run[rb], o[rb], lane);
      M::pv(o[rb], pk[0], buf + TILE + 32 * wave * ROWB, of, lane);
    }
  }
};

// ---------------------------------------------------------------------------------------
// Split-K decode: one workgroup = one (sequence, K/V head, key chunk). Its rows are the
// G * len_q (query head, query position) pairs of the group, shared by the 4 waves, so
// every K/V byte is read once for the whole group. Each 128-key stage gives each wave its
// own 32-key block; each wave keeps its own running state and writes its own partial
// (O_e normalised, LSE_e) with e = chunk * 4 + wave. The combine kernel merges partials.
// ---------------------------------------------------------------------------------------
template <typename T, int D, int NRB>
__global__ __launch_bounds__(256, 1) void fwd_splitk_kernel(FwdParams p) {
  typedef Mma<T, D> M;
  constexpr int BN = SPLITK_STAGE, ROWB = M::ROWB;
  constexpr int TILE = BN * ROWB;
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

  // Rows: r = position * G + head-in-group.
  typename M::QOperand qr[NRB][M::QREGS];
  int pq[NRB];
  bool rvalid[NRB];
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const int r = rb * 32 + (lane & 31);
    rvalid[rb] = r < R;
    pq[rb] = rvalid[rb] ? r / G : 0;
    const int h = kvh * G + (rvalid[rb] ? r % G : 0);
    const T* qrow = static_cast<const T*>(p.q) + ((size_t)(g.q_start + pq[rb]) * p.hq + h) * D;
    M::load_q(qr[rb], qrow, rvalid[rb], p.neg != 0, lane);
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
  DmaStager<ROWB, BN, 4> dma;
  dma.init(wave, lane, rstride);

  SplitkWave<T, D, NRB> st;
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
    st.stage(buf0, k0, klo, khi, R, wave, pq, g, p, qr, of, lane);
    wait_vmem();
    __syncthreads();
    if (it + 1 < nst) {
      if (it + 2 < nst) {
        dma.issue(kb0 + (size_t)(k0 + 2 * BN) * rstride, g.len_k - k0 - 2 * BN, rstride, buf0);
        dma.issue(vb0 + (size_t)(k0 + 2 * BN) * rstride, g.len_k - k0 - 2 * BN, rstride, buf0 + TILE);
      }
      st.stage(buf1, k0 + BN, klo, khi, R, wave, pq, g, p, qr, of, lane);
      wait_vmem();
      __syncthreads();
    }
  }
  f32x16 (&o)[NRB][D / 32] = st.o;
  float (&m_run)[NRB] = st.m_run;
  float (&l_run)[NRB] = st.l_run;

  // Partial of split e: normalised O_e (fp32) and LSE_e; empty -> O_e = 0, LSE_e = -inf.
  const int e = sigma * 4 + wave;
  const int hg = lane >> 5;
#pragma unroll
  for (int rb = 0; rb < NRB; ++rb) {
    const float lt = sum_halves(l_run[rb]);
    const bool nonempty = lt > 0.0f;
    const float inv = nonempty ? 1.0f / lt : 0.0f;
    if (!rvalid[rb]) continue;
    const int r = rb * 32 + (lane & 31);
    const int t = g.q_start + pq[rb];
    const int h = kvh * G + r % G;
    float* dst = p.part_o + (((size_t)e * p.total_q + t) * p.hq + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int d = db * 32 + 8 * a + 4 * hg;
        *reinterpret_cast<f32x4*>(dst + d) =
            f32x4{nonempty ? o[rb][db][4 * a] * inv : 0.0f, nonempty ? o[rb][db][4 * a + 1] * inv : 0.0f,
                  nonempty ? o[rb][db][4 * a + 2] * inv : 0.0f, nonempty ? o[rb][db][4 * a + 3] * inv : 0.0f};
      }
    if (hg == 0)
      p.part_lse[((size_t)e * p.hq + h) * p.total_q + t] =
          nonempty ? (m_run[rb] + fast_log2(lt)) * LN2 : neg_inf();
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
// Mask probe: the prefill kernel's decisions (stage range, per-wave block class, per-lane
// test) replayed for single (query token, key token) pairs.
// ---------------------------------------------------------------------------------------
__global__ void mask_probe_kernel(const int32_t* cu_q, const int32_t* cu_k, int num_seqs, int mode,
                                  int window, int q0, int nq, int k0, int nk, uint8_t* bits) {
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (long)nq * nk) return;
  const int t = q0 + (int)(idx / nk), u = k0 + (int)(idx % nk);
  const int s = seq_of_token(cu_q, num_seqs, t);
  const SeqGeom g = load_geom_lane(cu_q, cu_k, s, mode);
  const int pq = t - g.q_start;
  const int p0 = (pq / FWD_BM) * FWD_BM, p1 = min(p0 + FWD_BM, g.len_q);
  const int wp0 = p0 + ((pq - p0) / 32) * 32, wp1 = min(wp0 + 32, p1);
  int klo, khi;
  visible_keys(p0, p1, g, mode, window, klo, khi);
  const int kstart = (klo / FWD_BN) * FWD_BN;
  const int nst = khi > klo ? (khi - kstart + FWD_BN - 1) / FWD_BN : 0;
  uint8_t bit = 0;
  const int pk = u - g.k_start;
  if (u >= g.k_start && pk < g.len_k && pk >= kstart && pk < kstart + nst * FWD_BN) {
    const int kt = kstart + ((pk - kstart) / FWD_BN) * FWD_BN;
    const int cls = block_class(wp0, wp1, kt, kt + FWD_BN, g, mode, window);
    bit = cls == 2 ? 1 : (cls == 1 ? (pair_allowed(pq, pk, g, mode, window) ? 1 : 0) : 0);
  }
  bits[idx] = bit;
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
  p.c2 = (float)c2;
  p.neg = a.scale < 0;
  p.mode = a.mode;
  p.window = a.window;
  p.out = a.out;
  p.lse = a.lse;
  return p;
}

int fwd_prefill_grid(const FwdArgs& a) {
  const long nslots = (long)a.total_q / FWD_BM + a.num_seqs;
  const long nlogical = nslots * a.hq;
  return (int)(((nlogical + 7) / 8) * 8);
}

template <typename T, int D>
static hipError_t prefill_typed(const FwdArgs& a, hipStream_t st) {
  FwdParams p = make_params(a);
  p.nslots = a.total_q / FWD_BM + a.num_seqs;
  p.nlogical = p.nslots * a.hq;
  const int grid = fwd_prefill_grid(a);
  hipLaunchKernelGGL((fwd_prefill_kernel<T, D>), dim3(grid), dim3(256), 0, st, p);
  return hipGetLastError();
}

hipError_t launch_fwd_prefill(const FwdArgs& a, hipStream_t st) {
  if (a.dtype == 0) return a.d == 64 ? prefill_typed<__bf16, 64>(a, st) : prefill_typed<__bf16, 128>(a, st);
  return a.d == 64 ? prefill_typed<float, 64>(a, st) : prefill_typed<float, 128>(a, st);
}

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
  p.nsplit = nsb * 4;
  const size_t obytes = (size_t)p.nsplit * a.total_q * a.hq * D * sizeof(float);
  p.part_o = static_cast<float*>(ws);
  p.part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) + ((obytes + 255) / 256) * 256);
  const int grid = a.num_seqs * a.hkv * nsb;
  const int rows = (a.hq / a.hkv) * a.max_q;
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

hipError_t launch_mask_probe(const int32_t* cu_q, const int32_t* cu_k, int num_seqs, int mode,
                             int window, int q0, int nq, int k0, int nk, uint8_t* bits,
                             hipStream_t st) {
  const long n = (long)nq * nk;
  const int grid = (int)((n + 255) / 256);
  hipLaunchKernelGGL(mask_probe_kernel, dim3(grid), dim3(256), 0, st, cu_q, cu_k, num_seqs, mode,
                     window, q0, nq, k0, nk, bits);
  return hipGetLastError();
}

}  // namespace attn
