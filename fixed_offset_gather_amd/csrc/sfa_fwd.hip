// Forward kernels of libsfa (gfx950).
//
// fwd_offsets: causal attention over the window 0..W plus offsets shared by
// every query ("Depth-Staggered Fibonacci Spacing for Sparse Attention",
// key-set definition and gather paragraph; "Christoffel-Balanced Sparse
// Attention", pseudocode, with offsets as backward distances).  Because the
// offsets are shared, slot s of the BQ consecutive queries [i0, i0+BQ) reads
// the contiguous rows [i0-lo_s-1, i0+BQ-1-lo_s].  Slots are sorted by lo and
// grouped into stages whose row ranges fit CAP rows; each stage is staged
// once into LDS (K rotated to fp32 at its true position, V widened to fp32)
// with coalesced 16-byte loads and then serves every slot of the stage for
// all query heads of the KV group.
//
// Work split: one workgroup per (sequence, kv head, query block); LPQ lanes
// per query, each holding DC = D/LPQ dims of all G query heads of the group,
// so one LDS read of a key/value element feeds G FMAs.  Logits are reduced
// across the LPQ lanes with DPP (bf16: a reduce-scatter over the heads,
// after which each lane owns one head's softmax state; fp32: per-head sums,
// lane c owning head c % G); probabilities and rescale factors are
// broadcast back with DPP.  Online softmax in the log2 domain over chunks
// of SC slots.
//
// fwd_edges: attention over per-query edge lists ("Critical power-law
// sparse attention", item 2): rows are arbitrary, so keys are read straight
// from global memory (L2-resident) with the same lane layout.
#include "sfa_device.h"
#include "sfa_internal.h"
#include "sfa_launch.h"

namespace sfa {

constexpr int BQ = 64;   // queries per workgroup
constexpr int SC = 4;    // slots per online-softmax chunk
constexpr int ESC = 4;   // edges per chunk (keys come from global memory)

template <int D>
struct RowPad {
  static constexpr int value = D + 4;  // floats per LDS row (16-byte pad)
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* rope;
  int n, hq, hkv, nblk, tiles;
  int tiles_per_blk;  // sequences (batch x kv heads): tiles = nblk * this
  float scale_log2;   // scale * log2(e)
};

// Logit of lane's own head for one key chunk; `own` selects head c % G.
template <int G, int LPQ, int DC>
__device__ __forceinline__ float own_logit(const float (&qv)[G][DC], const float (&kt)[DC], int own) {
  float part[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float acc = 0.f;
#pragma unroll
    for (int x = 0; x < DC; ++x) acc = fmaf(qv[h][x], kt[x], acc);
    part[h] = group_sum<LPQ>(acc);
  }
  float mine = part[0];
#pragma unroll
  for (int h = 1; h < G; ++h) mine = (own == h) ? part[h] : mine;
  return mine;
}

// The same over raw bfloat16 pairs: v_dot2_f32_bf16, each product exact.
template <int G, int LPQ, int DW>
__device__ __forceinline__ float own_logit_bf(const uint32_t (&qb)[G][DW], const uint32_t (&kw)[DW], int own) {
  float part[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float acc = 0.f;
#pragma unroll
    for (int x = 0; x < DW; ++x) acc = dot2_bf(qb[h][x], kw[x], acc);
    part[h] = group_sum<LPQ>(acc);
  }
  float mine = part[0];
#pragma unroll
  for (int h = 1; h < G; ++h) mine = (own == h) ? part[h] : mine;
  return mine;
}

template <int G, int LPQ>
struct Bcast {
  template <int H = 0>
  static __device__ __forceinline__ void run(float x, float (&out)[G]) {
    if constexpr (H < G) {
      out[H] = owner_bcast<G, LPQ, H>(x);
      run<H + 1>(x, out);
    }
  }
};

template <typename T, int D, int G, int LPQ, int CAP, bool INTERP>
__global__ __launch_bounds__(BQ* LPQ) void fwd_offsets_kernel(FwdArgs a, SlotTable st) {
  constexpr int DC = D / LPQ;
  constexpr int KS = RowPad<D>::value;
  constexpr int E = 16 / sizeof(T);       // elements per 16-byte global chunk
  constexpr int CPR = D / E;              // chunks per row
  constexpr int NT = BQ * LPQ;
  static_assert(DC >= 2 && DC % 2 == 0, "lane chunk");
  __shared__ __align__(16) float Ks[CAP * KS];
  __shared__ __align__(16) float Vs[CAP * KS];

  const int tid = threadIdx.x;
  const int qq = tid / LPQ;
  const int c = tid % LPQ;
  const int own = c % G;
  const SeqBlock sb = lpt_seq_block(blockIdx.x, a.tiles, a.nblk);  // longest blocks first
  const int seq = sb.seq;
  const int blk = sb.blk;
  const int b = seq / a.hkv, g = seq % a.hkv;
  const int n = a.n;
  const int i0 = blk * BQ;
  const int i = i0 + qq;
  const bool active = i < n;
  const int i_last = min(i0 + BQ, n) - 1;

  // Slot table copied to LDS once: the hot loops read it with uniform
  // addresses instead of scalar loads from the kernel arguments.
  // (dynamic LDS of 3 x count words, so a short table takes little LDS)
  extern __shared__ __align__(16) int fwd_slot_smem[];
  int* const s_lo = fwd_slot_smem;
  float* const s_w = reinterpret_cast<float*>(fwd_slot_smem + st.count);
  float* const s_mult = reinterpret_cast<float*>(fwd_slot_smem + 2 * st.count);
  for (int t = threadIdx.x; t < st.count; t += blockDim.x) {
    s_lo[t] = st.s[t].lo;
    s_w[t] = st.s[t].frac;
    s_mult[t] = st.s[t].mult;
  }
  __syncthreads();

  const T* __restrict__ Q = static_cast<const T*>(a.q);
  const T* __restrict__ K = static_cast<const T*>(a.k);
  const T* __restrict__ V = static_cast<const T*>(a.v);

  // Rotated query chunk of every head in the group.
  float qv[G][DC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (active) {
      const T* src = Q + ((size_t(b) * n + i) * a.hq + size_t(g) * G + h) * D + c * DC;
      load_vec<DC>(src, qv[h]);
      if (a.rope) rotate_pairs<DC, 1>(qv[h], a.rope + size_t(i) * D, c * DC);
    } else {
#pragma unroll
      for (int x = 0; x < DC; ++x) qv[h][x] = 0.f;
    }
  }

  float o[G][DC];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int x = 0; x < DC; ++x) o[h][x] = 0.f;
  float m = neg_inf(), l = 0.f;

  const size_t kv_row = size_t(a.hkv) * D;                  // elements between rows
  const T* Kseq = K + size_t(b) * n * kv_row + size_t(g) * D;
  const T* Vseq = V + size_t(b) * n * kv_row + size_t(g) * D;

  int s = 0;
  const int S = st.count;
  while (s < S) {
    const int lo0 = st.s[s].lo;
    if (lo0 > i_last) break;  // this slot and all later ones are masked for the block
    int lomax = lo0 + ((INTERP && st.s[s].frac > 0.f) ? 1 : 0);
    int e = s + 1;
    while (e < S) {
      const int le = st.s[e].lo;
      if (le > i_last) break;
      const int need = max(lomax, le + ((INTERP && st.s[e].frac > 0.f) ? 1 : 0));
      if (need - lo0 + BQ > CAP) break;
      lomax = need;
      ++e;
    }
    const int r0 = i0 - lomax;          // absolute position of LDS row 0
    const int nrows = lomax - lo0 + BQ;

    __syncthreads();  // the previous stage is fully consumed
    for (int t = tid; t < nrows * CPR; t += NT) {
      const int row = t / CPR, cc = t % CPR;
      const int pos = r0 + row;
      float kf[E], vf[E];
      if (pos >= 0 && pos < n) {
        load_vec<E>(Kseq + size_t(pos) * kv_row + cc * E, kf);
        load_vec<E>(Vseq + size_t(pos) * kv_row + cc * E, vf);
        if (a.rope) rotate_pairs<E, 1>(kf, a.rope + size_t(pos) * D, cc * E);
      } else {
#pragma unroll
        for (int x = 0; x < E; ++x) kf[x] = vf[x] = 0.f;
      }
      store_vec<E>(Ks + row * KS + cc * E, kf);
      store_vec<E>(Vs + row * KS + cc * E, vf);
    }
    __syncthreads();

    for (int s0 = s; s0 < e; s0 += SC) {
      // The chunk's slot entries, read together (one wait for all of them).
      int lo_c[SC];
      float w_c[SC], mult_c[SC];
#pragma unroll
      for (int j = 0; j < SC; ++j) {
        const int sc = min(s0 + j, e - 1);
        lo_c[j] = s_lo[sc];
        w_c[j] = s_w[sc];
        mult_c[j] = s_mult[sc];
      }
      float sl[SC];
#pragma unroll
      for (int j = 0; j < SC; ++j) {
        sl[j] = neg_inf();
        const int sj = s0 + j;
        if (sj < e) {
          const int lo = __builtin_amdgcn_readfirstlane(lo_c[j]);
          const float w = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(w_c[j])));
          const int r = i - lo - r0;  // in [0, nrows) for every lane of the block
          float kt[DC];
          load_vec<DC>(Ks + r * KS + c * DC, kt);
          if (INTERP && w != 0.f) {
            float kb[DC];
            load_vec<DC>(Ks + (r - 1) * KS + c * DC, kb);
#pragma unroll
            for (int x = 0; x < DC; ++x) kt[x] = fmaf(w, kb[x] - kt[x], kt[x]);
          }
          const float mine = own_logit<G, LPQ, DC>(qv, kt, own);
          // the nearer row i - lo exists: mn <= i - lo <= n - 1 (as in the
          // bf16 kernel below)
          const int mn = w != 0.f ? 1 : 0;
          const bool valid = unsigned(i - lo - mn) < unsigned(n - mn);
          sl[j] = valid ? mine * a.scale_log2 : neg_inf();
        }
      }
      float mx = m;
#pragma unroll
      for (int j = 0; j < SC; ++j) mx = fmaxf(mx, sl[j]);
      // the reference moves only past kRescaleSlack (one ballot per chunk)
      if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleSlack) != 0) {
        const float mr = (mx == neg_inf()) ? 0.f : mx;
        const float corr = __builtin_amdgcn_exp2f(m - mr);
        l *= corr;
        m = mx;
        float ch[G];
        Bcast<G, LPQ>::run(corr, ch);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int x = 0; x < DC; ++x) o[h][x] *= ch[h];
      }
      const float mref = (m == neg_inf()) ? 0.f : m;
      float p[SC];
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < SC; ++j) {
        // a slot past the stage has sl = -inf, so p = 0 whatever its
        // (clamped) multiplicity: no per-slot condition
        p[j] = __builtin_amdgcn_exp2f(sl[j] - mref) * mult_c[j];
        ps += p[j];
      }
      l += ps;
#pragma unroll
      for (int j = 0; j < SC; ++j) {
        const int sj = s0 + j;
        if (sj < e) {
          const int lo = __builtin_amdgcn_readfirstlane(s_lo[sj]);
          const float w = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(s_w[sj])));
          const int r = i - lo - r0;
          float vt[DC];
          load_vec<DC>(Vs + r * KS + c * DC, vt);
          if (INTERP && w != 0.f) {
            float vb[DC];
            load_vec<DC>(Vs + (r - 1) * KS + c * DC, vb);
#pragma unroll
            for (int x = 0; x < DC; ++x) vt[x] = fmaf(w, vb[x] - vt[x], vt[x]);
          }
          float ph[G];
          Bcast<G, LPQ>::run(p[j], ph);
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int x = 0; x < DC; ++x) o[h][x] = fmaf(ph[h], vt[x], o[h][x]);
        }
      }
    }
    s = e;
  }

  float lh[G];
  Bcast<G, LPQ>::run(l, lh);
  if (active) {
    T* O = static_cast<T*>(a.o);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float inv = 1.f / lh[h];
      float out[DC];
#pragma unroll
      for (int x = 0; x < DC; ++x) out[x] = o[h][x] * inv;
      store_vec<DC>(O + ((size_t(b) * n + i) * a.hq + size_t(g) * G + h) * D + c * DC, out);
    }
    if (a.lse && c < G) a.lse[(size_t(b) * a.hq + size_t(g) * G + c) * n + i] = (m + log2f(l)) * kLn2;
  }
}

// bf16 tensors: the same algorithm with f16 operands.  LDS holds K rotated
// at its true position and V, both as packed f16 (half the footprint of
// fp32 rows, so more workgroups fit on a CU); the query is rotated, scaled
// by scale*log2(e) and packed to f16 once.  Logits use v_dot2_f32_f16 (two
// f16 products per instruction, fp32 accumulation), interpolation is packed
// f16 arithmetic, and each value element is widened to fp32 once and feeds
// fp32 FMAs for all G heads.  The softmax and the output accumulation stay
// in fp32.  Register j of a lane holds head HeadSlice::head(c, j), so the
// per-slot logit is a reduce-scatter (each lane ends with its own head's
// sum) and p is spread back with G - 1 DPP moves; BQH queries per
// workgroup.  RAWK (integer offsets without rotation): K rows are staged as
// the bf16 input words, unconverted, the query is packed as bf16 pairs
// (exact) and the logits use v_dot2_f32_bf16, whose products are exact, then
// take scale*log2(e) after the sum (Christoffel forward 84.1 -> 81.1 us).
template <int D, int G, int LPQ, int BQH, int CAP, bool INTERP, bool RAWK>
__global__ __launch_bounds__(BQH* LPQ) void fwd_offsets_h16_kernel(FwdArgs a, SlotTable st) {
  static_assert(!(RAWK && INTERP), "raw bf16 K rows are not interpolated");
  constexpr int DC = D / LPQ;  // dims per lane
  constexpr int DW = DC / 2;   // f16 pairs per lane
  constexpr int RW = D / 2 + 4;  // 32-bit words per LDS row (16-byte pad)
  constexpr int CPR = D / 8;     // 16-byte global chunks (8 bf16) per row
  constexpr int NT = BQH * LPQ;
  static_assert(DC >= 2 && DC % 2 == 0, "lane chunk");
  using HS = HeadSlice<G, LPQ>;
  // K and V rows of a stage in one LDS array, each led by a pad row:
  // [pad][K rows 0..CAP-1][pad][V rows 0..CAP-1].  Row r - 1 of a slot (its
  // interpolation partner, or a pad row when r = 0) is never below the
  // array, and the four rows a slot reads lie at fixed byte offsets from it,
  // so one address per slot serves all of them.
  constexpr int VOFF = (CAP + 1) * RW;  // words from a K row to the same V row
  static_assert((VOFF + RW) * 4 < 65536, "row offsets fit a ds_read offset");
  __shared__ __align__(16) uint32_t KV[(2 * CAP + 2) * RW];
  uint32_t* const Ks = KV + RW;
  uint32_t* const Vs = Ks + VOFF;

  const int tid = threadIdx.x;
  const int qq = tid / LPQ;
  const int c = tid % LPQ;
  const int own = HS::own(c);
  const SeqBlock sb = lpt_seq_block(blockIdx.x, a.tiles, a.nblk);  // longest blocks first
  const int seq = sb.seq;
  const int blk = sb.blk;
  const int b = seq / a.hkv, g = seq % a.hkv;
  const int n = a.n;
  const int i0 = blk * BQH;
  const int i = i0 + qq;
  const bool active = i < n;
  const int i_last = min(i0 + BQH, n) - 1;

  // Slot table copied to LDS once: the hot loops read it with uniform
  // addresses instead of scalar loads from the kernel arguments.
  // The fraction is kept as its bit pattern: frac is +0 or positive, so the
  // bits read as a non-negative integer decide interpolation with scalar
  // integer operations.
  // (dynamic LDS of 3 x count words: the page-1 table takes 312 bytes, so
  // four workgroups still share a CU)
  extern __shared__ __align__(16) int fwd_slot_smem[];
  int* const s_lo = fwd_slot_smem;
  int* const s_wb = fwd_slot_smem + st.count;
  float* const s_mult = reinterpret_cast<float*>(fwd_slot_smem + 2 * st.count);
  for (int t = threadIdx.x; t < st.count; t += blockDim.x) {
    s_lo[t] = st.s[t].lo;
    s_wb[t] = __float_as_int(st.s[t].frac);
    s_mult[t] = st.s[t].mult;
  }
  __syncthreads();

  const bf16_t* __restrict__ Q = static_cast<const bf16_t*>(a.q);
  const bf16_t* __restrict__ K = static_cast<const bf16_t*>(a.k);
  const bf16_t* __restrict__ V = static_cast<const bf16_t*>(a.v);

  // Register j of a lane holds head HS::head(c, j) of the group.
  uint32_t qh[G][DW];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float qf[DC];
    if (active) {
      load_vec<DC>(Q + ((size_t(b) * n + i) * a.hq + size_t(g) * G + HS::head(c, h)) * D + c * DC, qf);
      if (a.rope) rotate_pairs<DC, 1>(qf, a.rope + size_t(i) * D, c * DC);
    } else {
#pragma unroll
      for (int x = 0; x < DC; ++x) qf[x] = 0.f;
    }
#pragma unroll
    for (int x = 0; x < DW; ++x)
      qh[h][x] = RAWK ? pack_bf2(qf[2 * x], qf[2 * x + 1])
                      : pack_h2(qf[2 * x] * a.scale_log2, qf[2 * x + 1] * a.scale_log2);
  }

  float o[G][DC];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int x = 0; x < DC; ++x) o[h][x] = 0.f;
  float m = neg_inf(), l = 0.f;

  const size_t kv_row = size_t(a.hkv) * D;
  const bf16_t* Kseq = K + size_t(b) * n * kv_row + size_t(g) * D;
  const bf16_t* Vseq = V + size_t(b) * n * kv_row + size_t(g) * D;

  int s = 0;
  const int S = st.count;
  while (s < S) {
    const int lo0 = st.s[s].lo;
    if (lo0 > i_last) break;
    int lomax = lo0 + ((INTERP && st.s[s].frac > 0.f) ? 1 : 0);
    int e = s + 1;
    while (e < S) {
      const int le = st.s[e].lo;
      if (le > i_last) break;
      const int need = max(lomax, le + ((INTERP && st.s[e].frac > 0.f) ? 1 : 0));
      if (need - lo0 + BQH > CAP) break;
      lomax = need;
      ++e;
    }
    const int r0 = i0 - lomax;
    const int nrows = lomax - lo0 + BQH;

    __syncthreads();
    for (int t = tid; t < nrows * CPR; t += NT) {
      const int row = t / CPR, cc = t % CPR;
      const int pos = r0 + row;
      float kf[8], vf[8];
      uint4 kraw = make_uint4(0, 0, 0, 0);
      if (pos >= 0 && pos < n) {
        if constexpr (RAWK) {
          kraw = *reinterpret_cast<const uint4*>(Kseq + size_t(pos) * kv_row + cc * 8);
        } else {
          load_vec<8>(Kseq + size_t(pos) * kv_row + cc * 8, kf);
          if (a.rope) rotate_pairs<8, 1>(kf, a.rope + size_t(pos) * D, cc * 8);
        }
        load_vec<8>(Vseq + size_t(pos) * kv_row + cc * 8, vf);
      } else {
#pragma unroll
        for (int x = 0; x < 8; ++x) kf[x] = vf[x] = 0.f;
      }
      if constexpr (RAWK)
        *reinterpret_cast<uint4*>(Ks + row * RW + cc * 4) = kraw;
      else
        *reinterpret_cast<uint4*>(Ks + row * RW + cc * 4) =
            make_uint4(pack_h2(kf[0], kf[1]), pack_h2(kf[2], kf[3]), pack_h2(kf[4], kf[5]), pack_h2(kf[6], kf[7]));
      *reinterpret_cast<uint4*>(Vs + row * RW + cc * 4) =
          make_uint4(pack_h2(vf[0], vf[1]), pack_h2(vf[2], vf[3]), pack_h2(vf[4], vf[5]), pack_h2(vf[6], vf[7]));
    }
    __syncthreads();

    // K row r - 1 of the slot at lo = 0; a slot's rows are lo rows earlier.
    const uint32_t* const lane_kv = Ks + (i - r0 - 1) * RW + c * DW;
    for (int s0 = s; s0 < e; s0 += SC) {
      // The chunk's slot entries, read together (one wait for all of them
      // instead of one before each slot's row reads).
      int lo_c[SC], wb_c[SC];
      float mult_c[SC];
#pragma unroll
      for (int j = 0; j < SC; ++j) {
        const int sc = min(s0 + j, e - 1);
        lo_c[j] = s_lo[sc];
        wb_c[j] = s_wb[sc];
        mult_c[j] = s_mult[sc];
      }
      float sl[SC];
#pragma unroll
      for (int j = 0; j < SC; ++j) {
        sl[j] = neg_inf();
        const int sj = s0 + j;
        if (sj < e) {
          const int lo = __builtin_amdgcn_readfirstlane(lo_c[j]);
          const int wbits = __builtin_amdgcn_readfirstlane(wb_c[j]);
          const uint32_t* const kp = lane_kv - lo * RW;  // K row r - 1
          uint32_t kw[DW];
          load_words<DW>(kp + RW, kw);
          if (INTERP && wbits != 0) {
            uint32_t kb[DW];
            load_words<DW>(kp, kb);
            const float w = __int_as_float(wbits);
            const half2_t w2 = {(_Float16)w, (_Float16)w};
#pragma unroll
            for (int x = 0; x < DW; ++x) kw[x] = lerp_h2(kw[x], kb[x], w2);
          }
          // Per-head partial dots, summed over the query's lanes as a
          // reduce-scatter: each lane ends with its own head's logit.
          float part[G];
#pragma unroll
          for (int h = 0; h < G; ++h) {
            float acc = 0.f;
#pragma unroll
            for (int x = 0; x < DW; ++x) acc = RAWK ? dot2_bf(qh[h][x], kw[x], acc) : dot2_h(qh[h][x], kw[x], acc);
            part[h] = acc;
          }
          const float mine = RAWK ? HS::reduce(part) * a.scale_log2 : HS::reduce(part);
          // The nearer row i - lo exists (i >= lo + frac, and below n for a
          // negative offset): mn <= i - lo <= n - 1 with mn = 1 for an
          // interpolated slot (integer arithmetic on the fraction's bits,
          // so it stays scalar), one unsigned compare.  Queries past n have
          // zero q; their state stays finite and is never stored.
          const int mn = INTERP ? min(wbits, 1) : 0;
          const bool valid = unsigned(i - lo - mn) < unsigned(n - mn);
          sl[j] = valid ? mine : neg_inf();
        }
      }
      float mx = m;
#pragma unroll
      for (int j = 0; j < SC; ++j) mx = fmaxf(mx, sl[j]);
      // the reference moves only past kRescaleSlack (one ballot per chunk)
      if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleSlack) != 0) {
        const float mr = (mx == neg_inf()) ? 0.f : mx;
        const float corr = __builtin_amdgcn_exp2f(m - mr);
        l *= corr;
        m = mx;
        float ch[G];
        HS::bcast(corr, ch);
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
          for (int x = 0; x < DC; ++x) o[h][x] *= ch[h];
      }
      const float mref = (m == neg_inf()) ? 0.f : m;
      float p[SC];
      float ps = 0.f;
#pragma unroll
      for (int j = 0; j < SC; ++j) {
        // a slot past the stage has sl = -inf, so p = 0 whatever its
        // (clamped) multiplicity: no per-slot condition
        p[j] = __builtin_amdgcn_exp2f(sl[j] - mref) * mult_c[j];
        ps += p[j];
      }
      l += ps;
#pragma unroll
      for (int j = 0; j < SC; ++j) {
        const int sj = s0 + j;
        if (sj < e) {
          const int lo = __builtin_amdgcn_readfirstlane(lo_c[j]);
          const int wbits = __builtin_amdgcn_readfirstlane(wb_c[j]);
          const uint32_t* const kp = lane_kv - lo * RW;  // K row r - 1
          float ph[G];
          HS::bcast(p[j], ph);
          uint32_t vw[DW];
          load_words<DW>(kp + RW + VOFF, vw);
          if (INTERP && wbits != 0) {
            uint32_t vb[DW];
            load_words<DW>(kp + VOFF, vb);
            const float w = __int_as_float(wbits);
            const half2_t w2 = {(_Float16)w, (_Float16)w};
#pragma unroll
            for (int x = 0; x < DW; ++x) vw[x] = lerp_h2(vw[x], vb[x], w2);
          }
          // With G >= 2 heads each value element is widened to fp32 once
          // and then feeds G plain fp32 FMAs; the empty asm keeps the
          // widening from being folded back into G mixed-precision FMAs,
          // which issue at half the rate.  With one head the element feeds
          // one FMA, and the folded form (one v_fma_mix_f32 instead of a
          // conversion and an FMA) is the cheaper one.
          float vf[DC];
#pragma unroll
          for (int x = 0; x < DW; ++x) {
            vf[2 * x] = float(as_h2(vw[x]).x);
            vf[2 * x + 1] = float(as_h2(vw[x]).y);
            if constexpr (G >= 2) asm volatile("" : "+v"(vf[2 * x]), "+v"(vf[2 * x + 1]));
          }
#pragma unroll
          for (int h = 0; h < G; ++h)
#pragma unroll
            for (int x = 0; x < DC; ++x) o[h][x] = fmaf(ph[h], vf[x], o[h][x]);
        }
      }
    }
    s = e;
  }

  float lh[G];
  HS::bcast(l, lh);
  if (active) {
    bf16_t* O = static_cast<bf16_t*>(a.o);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float inv = 1.f / lh[h];
      float out[DC];
#pragma unroll
      for (int x = 0; x < DC; ++x) out[x] = o[h][x] * inv;
      store_vec<DC>(O + ((size_t(b) * n + i) * a.hq + size_t(g) * G + HS::head(c, h)) * D + c * DC, out);
    }
    if (a.lse && HS::writer(c))
      a.lse[(size_t(b) * a.hq + size_t(g) * G + own) * n + i] = (m + log2f(l)) * kLn2;
  }
}

// ------------------------------------------------------------ edge lists

struct EdgeArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const float* rope;
  const int32_t* edges;
  const int32_t* count;
  int n, hq, hkv, nblk, tiles, width;
  float scale_log2;
};

// RAWK (bf16 without rotation): the query and the listed K and V rows stay
// bf16 words; the logits use v_dot2_f32_bf16 (exact products), and a chunk's
// V rows are requested together with its K rows, so the chunk waits for
// memory once instead of twice (power-law forward 26.8 -> 24.8 us).
template <typename T, int D, int G, int LPQ, bool RAWK>
__global__ __launch_bounds__(BQ* LPQ) void fwd_edges_kernel(EdgeArgs a) {
  static_assert(!RAWK || sizeof(T) == 2, "raw rows are bf16");
  constexpr int DC = D / LPQ;
  constexpr int DW = DC / 2;
  const int tid = threadIdx.x;
  const int qq = tid / LPQ;
  const int c = tid % LPQ;
  const int own = c % G;
  const int tile = xcd_tile(blockIdx.x, a.tiles);
  const int seq = tile / a.nblk;
  const int blk = tile % a.nblk;
  const int b = seq / a.hkv, g = seq % a.hkv;
  const int n = a.n;
  const int i = blk * BQ + qq;
  const bool active = i < n;

  const T* __restrict__ Q = static_cast<const T*>(a.q);
  const T* __restrict__ K = static_cast<const T*>(a.k);
  const T* __restrict__ V = static_cast<const T*>(a.v);
  const size_t kv_row = size_t(a.hkv) * D;
  const T* Kseq = K + size_t(b) * n * kv_row + size_t(g) * D + c * DC;
  const T* Vseq = V + size_t(b) * n * kv_row + size_t(g) * D + c * DC;

  float qv[G][DC];
  uint32_t qb[G][DW];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    const size_t qoff = ((size_t(b) * n + i) * a.hq + size_t(g) * G + h) * D + c * DC;
    if constexpr (RAWK) {
      if (active) {
        load_words<DW>(reinterpret_cast<const uint32_t*>(Q + qoff), qb[h]);
      } else {
#pragma unroll
        for (int x = 0; x < DW; ++x) qb[h][x] = 0u;
      }
    } else if (active) {
      load_vec<DC>(Q + qoff, qv[h]);
      if (a.rope) rotate_pairs<DC, 1>(qv[h], a.rope + size_t(i) * D, c * DC);
    } else {
#pragma unroll
      for (int x = 0; x < DC; ++x) qv[h][x] = 0.f;
    }
  }
  const int cnt = active ? min(a.count[i], a.width) : 0;
  // Wave-uniform trip count: the largest list in the wavefront.
  int cmax = cnt;
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) cmax = max(cmax, __shfl_xor(cmax, msk));
  const int32_t* erow = a.edges + size_t(active ? i : 0) * a.width;

  float o[G][DC];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int x = 0; x < DC; ++x) o[h][x] = 0.f;
  float m = neg_inf(), l = 0.f;

  // The list entries of a chunk are read one chunk ahead, so the index
  // loads leave the chunk's dependency chain (index, then K row, then
  // logit).  An entry index is clamped to the width: a chunk can run past
  // it when the width is not a multiple of ESC.
  int keys[ESC];
#pragma unroll
  for (int j = 0; j < ESC; ++j) keys[j] = erow[min(j, a.width - 1)];
  for (int t0 = 0; t0 < cmax; t0 += ESC) {
    // Branch-free over the lanes' different lists: an entry past the
    // query's count or a padding entry reads row 0 (row 0 exists) and is
    // masked by its logit, so p = 0 for it.
    int knext[ESC];
#pragma unroll
    for (int j = 0; j < ESC; ++j) knext[j] = erow[min(t0 + ESC + j, a.width - 1)];
    float sl[ESC];
    int jj[ESC];
    uint32_t vraw[RAWK ? ESC : 1][DW];
    if constexpr (RAWK) {
      uint32_t kw[ESC][DW];
#pragma unroll
      for (int j = 0; j < ESC; ++j) {
        const int t = t0 + j;
        const int key = keys[j];
        const bool valid = t < cnt && key >= 0 && key < n;
        jj[j] = valid ? key : 0;
        load_words<DW>(reinterpret_cast<const uint32_t*>(Kseq + size_t(jj[j]) * kv_row), kw[j]);
        load_words<DW>(reinterpret_cast<const uint32_t*>(Vseq + size_t(jj[j]) * kv_row), vraw[j]);
        sl[j] = valid ? 0.f : neg_inf();
      }
#pragma unroll
      for (int j = 0; j < ESC; ++j) sl[j] += own_logit_bf<G, LPQ, DW>(qb, kw[j], own) * a.scale_log2;
    } else {
#pragma unroll
      for (int j = 0; j < ESC; ++j) {
        const int t = t0 + j;
        const int key = keys[j];
        const bool valid = t < cnt && key >= 0 && key < n;
        jj[j] = valid ? key : 0;
        float kt[DC];
        load_vec<DC>(Kseq + size_t(jj[j]) * kv_row, kt);
        if (a.rope) rotate_pairs<DC, 1>(kt, a.rope + size_t(jj[j]) * D, c * DC);
        const float mine = own_logit<G, LPQ, DC>(qv, kt, own);
        sl[j] = valid ? mine * a.scale_log2 : neg_inf();
      }
    }
    float mx = m;
#pragma unroll
    for (int j = 0; j < ESC; ++j) mx = fmaxf(mx, sl[j]);
    // the reference moves only past kRescaleSlack (one ballot per chunk)
    if (__builtin_amdgcn_ballot_w64(mx > m + kRescaleSlack) != 0) {
      const float mr = (mx == neg_inf()) ? 0.f : mx;
      const float corr = __builtin_amdgcn_exp2f(m - mr);
      l *= corr;
      m = mx;
      float ch[G];
      Bcast<G, LPQ>::run(corr, ch);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int x = 0; x < DC; ++x) o[h][x] *= ch[h];
    }
    const float mref = (m == neg_inf()) ? 0.f : m;
    float p[ESC];
    float ps = 0.f;
#pragma unroll
    for (int j = 0; j < ESC; ++j) {
      p[j] = __builtin_amdgcn_exp2f(sl[j] - mref);
      ps += p[j];
    }
    l += ps;
#pragma unroll
    for (int j = 0; j < ESC; ++j) {
      float vt[DC];
      if constexpr (RAWK) {
#pragma unroll
        for (int x = 0; x < DW; ++x) {
          vt[2 * x] = bf16_lo(vraw[j][x]);
          vt[2 * x + 1] = bf16_hi(vraw[j][x]);
        }
      } else {
        load_vec<DC>(Vseq + size_t(jj[j]) * kv_row, vt);  // p[j] = 0 for a masked entry
      }
      float ph[G];
      Bcast<G, LPQ>::run(p[j], ph);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int x = 0; x < DC; ++x) o[h][x] = fmaf(ph[h], vt[x], o[h][x]);
    }
#pragma unroll
    for (int j = 0; j < ESC; ++j) keys[j] = knext[j];
  }

  float lh[G];
  Bcast<G, LPQ>::run(l, lh);
  if (active) {
    T* O = static_cast<T*>(a.o);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float inv = lh[h] > 0.f ? 1.f / lh[h] : 0.f;
      float out[DC];
#pragma unroll
      for (int x = 0; x < DC; ++x) out[x] = o[h][x] * inv;
      store_vec<DC>(O + ((size_t(b) * n + i) * a.hq + size_t(g) * G + h) * D + c * DC, out);
    }
    if (a.lse && c < G)
      a.lse[(size_t(b) * a.hq + size_t(g) * G + c) * n + i] = l > 0.f ? (m + log2f(l)) * kLn2 : neg_inf();
  }
}

// ---------------------------------------------------------------- launch

namespace {

constexpr int kCap = 128;  // staged rows per stage (BQ + 64)

template <int D, int G>
constexpr int fwd_lpq() {
  // At least one lane per head of the group and at most 16 dims per lane.
  return G > D / 16 ? G : D / 16;
}

// f16 kernel: lanes per query and queries per workgroup (256 threads at
// most, 64 queries at most).  At least two lanes per head: with one lane
// per head (the whole group reduced by a full permutation of the lanes'
// registers) the page-1 layer measured slower than plain per-head sums
// (83.5 against 80.9 us), with two it is faster (77.6 us, 8 lanes of 8 dims
// at G = 4); at most 16 lanes and at least 2 dims per lane.
template <int D, int G>
constexpr int fwd_h16_lpq() {
  constexpr int want = 2 * G > D / 16 ? 2 * G : D / 16;
  constexpr int cap = D / 2 < 16 ? D / 2 : 16;
  return want < cap ? want : cap;
}
template <int D, int G>
constexpr int fwd_h16_bq() {
  return fwd_h16_lpq<D, G>() >= 8 ? 256 / fwd_h16_lpq<D, G>() : 64;
}

template <typename T, int D, int G, bool INTERP>
void launch_fwd_offsets_i(const SlotTable& t, const FwdArgs& a0, hipStream_t st) {
  if constexpr (sizeof(T) == 2) {
    constexpr int LPQ = fwd_h16_lpq<D, G>();
    constexpr int BQH = fwd_h16_bq<D, G>();
    static_assert(BQH + 64 <= kCap, "stage capacity");
    FwdArgs a = a0;
    a.nblk = (a.n + BQH - 1) / BQH;
    a.tiles = a.nblk * a.tiles_per_blk;
    // Integer offsets without rotation read the bf16 K rows as they are.
    if (!INTERP && a.rope == nullptr)
      SFA_LAUNCH((fwd_offsets_h16_kernel<D, G, LPQ, BQH, kCap, false, true>),
                         dim3(a.tiles), dim3(BQH * LPQ), 3 * 4 * t.count, st, a, t);
    else
      SFA_LAUNCH((fwd_offsets_h16_kernel<D, G, LPQ, BQH, kCap, INTERP, false>),
                         dim3(a.tiles), dim3(BQH * LPQ), 3 * 4 * t.count, st, a, t);
  } else {
    constexpr int LPQ = fwd_lpq<D, G>();
    const FwdArgs& a = a0;
    SFA_LAUNCH((fwd_offsets_kernel<T, D, G, LPQ, kCap, INTERP>), dim3(a.tiles), dim3(BQ * LPQ),
                       3 * 4 * t.count, st, a,
                       t);
  }
}

// The integer instantiation (no interpolation code) runs when every slot
// has frac == 0, unless SFA_FLAG_INTERP_KERNEL asks for the interpolating
// one; both give the same bits there.
template <typename T, int D, int G>
int launch_fwd_offsets_t(const Problem& p, const SlotTable& t, const FwdArgs& a, hipStream_t st) {
  bool interp = (p.flags & SFA_FLAG_INTERP_KERNEL) != 0;
  for (int s = 0; s < t.count && !interp; ++s) interp = t.s[s].frac > 0.f;
  if (interp)
    launch_fwd_offsets_i<T, D, G, true>(t, a, st);
  else
    launch_fwd_offsets_i<T, D, G, false>(t, a, st);
  return int(hipGetLastError());
}

template <typename T, int D, int G>
int launch_fwd_edges_t(const EdgeArgs& a, hipStream_t st) {
  constexpr int LPQ = fwd_lpq<D, G>();
  if constexpr (sizeof(T) == 2) {
    if (a.rope == nullptr) {  // bf16 without rotation: raw rows
      SFA_LAUNCH((fwd_edges_kernel<T, D, G, LPQ, true>), dim3(a.tiles), dim3(BQ * LPQ), 0, st, a);
      return int(hipGetLastError());
    }
  }
  SFA_LAUNCH((fwd_edges_kernel<T, D, G, LPQ, false>), dim3(a.tiles), dim3(BQ * LPQ), 0, st, a);
  return int(hipGetLastError());
}

// Calls F<T, D, G>(args...) for the runtime (dtype, D, G).
#define SFA_DISPATCH(FN, P, ...)                                                      \
  do {                                                                                \
    const int d_ = (P).D, g_ = (P).G;                                                 \
    if ((P).dtype == SFA_BF16) {                                                      \
      if (d_ == 128) SFA_DISPATCH_G(bf16_t, 128, FN, g_, __VA_ARGS__); /* bf16 only */ \
      SFA_DISPATCH_D(bf16_t, FN, d_, g_, __VA_ARGS__);                                \
    } else {                                                                          \
      SFA_DISPATCH_D(float, FN, d_, g_, __VA_ARGS__);                                 \
    }                                                                                 \
  } while (0)
#define SFA_DISPATCH_D(T, FN, d_, g_, ...)                                            \
  do {                                                                                \
    if (d_ == 64) SFA_DISPATCH_G(T, 64, FN, g_, __VA_ARGS__);                         \
    else if (d_ == 32) SFA_DISPATCH_G(T, 32, FN, g_, __VA_ARGS__);                    \
    else SFA_DISPATCH_G(T, 16, FN, g_, __VA_ARGS__);                                  \
  } while (0)
#define SFA_DISPATCH_G(T, D_, FN, g_, ...)                                            \
  do {                                                                                \
    if (g_ == 1) return FN<T, D_, 1>(__VA_ARGS__);                                    \
    if (g_ == 2) return FN<T, D_, 2>(__VA_ARGS__);                                    \
    if (g_ == 4) return FN<T, D_, 4>(__VA_ARGS__);                                    \
    return FN<T, D_, 8>(__VA_ARGS__);                                                 \
  } while (0)

}  // namespace

int launch_fwd_offsets(const Problem& p, const SlotTable& t, const void* q, const void* k, const void* v,
                       void* o, float* lse, void* stream) {
  FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.rope = p.rope;
  a.n = p.n;
  a.hq = p.hq;
  a.hkv = p.hkv;
  a.nblk = (p.n + BQ - 1) / BQ;
  a.tiles_per_blk = p.B * p.hkv;
  a.tiles = a.nblk * a.tiles_per_blk;
  a.scale_log2 = p.scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  SFA_DISPATCH(launch_fwd_offsets_t, p, p, t, a, st);
}

int launch_fwd_edges(const Problem& p, const int32_t* edges, const int32_t* count, int width, const void* q,
                     const void* k, const void* v, void* o, float* lse, void* stream) {
  EdgeArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.lse = lse;
  a.rope = p.rope;
  a.edges = edges;
  a.count = count;
  a.n = p.n;
  a.hq = p.hq;
  a.hkv = p.hkv;
  a.nblk = (p.n + BQ - 1) / BQ;
  a.tiles = a.nblk * p.B * p.hkv;
  a.width = width;
  a.scale_log2 = p.scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  SFA_DISPATCH(launch_fwd_edges_t, p, a, st);
}

}  // namespace sfa
