// Backward kernels of libsfa (gfx950) for L = <O, dO> of the window plus
// shared-offset forward.  Because every rung is a lerp of rows i-lo and
// i-lo-1, the output is differentiable in the rung distance, and through
// d_k = alpha f_k and the sigmoid map in theta ("Depth-Staggered Fibonacci
// Spacing for Sparse Attention", gather paragraph and alpha
// parameterisation).
//
// Launches on one stream, no atomics, fixed summation order:
//
// bwd_query (query-centric, same staging as the forward): recomputes each
//   logit, p = exp(logit - lse) and dp = dO.v~ in one pass over the slots.
//   Dvec = rowsum(dO*O) is formed exactly as sum_slots p dp (not from the
//   rounded forward output), and dq~ = scale sum p (dp - Dvec) k~ is
//   accumulated as scale (sum p dp k~ - Dvec sum p k~), then rotated back to
//   dQ.  The per-slot dot sums over a query's lanes are a reduce-scatter
//   over the heads (HeadSlice).  Every p is taken relative to l = sum_slots
//   p (1 up to the forward's lse, whose f16 logits are off by an amount
//   that grows with the logits): dQ, Dvec and, through 1/l stored beside p,
//   the key pass use p / l, the softmax of the fp32 logits.  p (0 where the
//   slot has no row), dp, Dvec / l and 1/l of every (query, slot, head) go
//   to the workspace.  The offset
//   gradient is formed here too, from the fp32 rows and weights: for rung k
//   and query head (i, h), dd_k gets scale dS (q~ . dK) + p (dO . dV) with
//   dK = Kr[i-lo-1] - Kr[i-lo] and dV likewise; written as
//   Y - Dvec X (Y = p (scale dp sd + vd), X = scale p sd) so that the
//   per-rung values wait in registers until Dvec is known, then summed over
//   the workgroup into one partial per (rung, workgroup).
// bwd_key (key-centric transpose gather): key j receives from query j+lo
//   (weight 1-frac) and j+lo+1 (weight frac) of every slot; those queries
//   form contiguous ranges, so each lane gathers instead of scattering.
//   fp32: one kernel; dK uses the relative rotation R(j)^T R(i) = R(i-j)
//   with i-j fixed per (slot, tap), so unrotated Q rows are combined first
//   and rotated once.  bf16: one launch of dK and dV workgroups (both in
//   one workgroup with one head per KV head) staging query rows into an LDS
//   ring of rows that consecutive stages share; with dd or dtheta asked,
//   a leading workgroup of the same launch does the reduction below.
// The dd reduction (reduce_body; a kernel of its own, bwd_reduce, for the
//   fp32 backward): sums the partials in block order (in double);
//   dalpha = sum f_k dd_k; dtheta = (alpha - 1/2)(3/2 - alpha) dalpha.
// The edge-list backward (bwd_edges_query, bwd_edges_key, further below)
// does the same per query and per key over explicit lists.
#include <cstring>

#include "sfa_device.h"
#include "sfa_internal.h"
#include "sfa_launch.h"

namespace sfa {

namespace {

constexpr int kCap = 128;

// Dims per key-pass tile (and per chunk of a packed key-pass row).
constexpr int key_chunk(int D) { return D >= 16 ? 16 : D; }
// Dims per bf16 key-pass tile (and per chunk of the packed rows the query
// pass writes).  With four or more heads per KV head, 32 dims: each of a
// key's chunk tiles loads and converts the same step weights, so wider
// tiles do that work for more dims (page-1 key pass 80.1 -> 78.7 us at 8
// waves per CU instead of 16).  With fewer heads 16: 32-dim tiles at one
// head per KV head were measured slower (Christoffel key pass 199 ->
// 263 us).
constexpr int key_chunk_h16(int D, int G) { return G >= 4 && D >= 32 ? 32 : key_chunk(D); }

// Queries per bwd_query workgroup and rows per stage.  With fewer than 4
// heads per KV head, 8-lane queries in blocks of 64 (8 waves) with 128-row
// stages: two workgroups share a CU (Christoffel query pass 210 -> 163 us
// against 32-query blocks).  With G >= 4 a query takes 16 lanes, and blocks
// of 16 queries (4 waves) with 72-row stages (30.6 KB of LDS) put four
// workgroups on a CU: the same 16 waves as two of 32 queries with 128-row
// stages, in workgroups half as long, so the launch's tail (the CUs left
// idle while its last workgroups finish) is half as long too (page-1 query
// pass 155.4 -> 148.9 us; 64 queries: 124 -> 142 us in an earlier build).
template <int G>
constexpr int bwd_bq() {
  return G >= 4 ? 16 : 64;
}
// Rows per stage: 72 with G >= 4 (four 16-query workgroups per CU).  With
// fewer heads, as many as let two 64-query workgroups share the 160 KiB of
// LDS: bf16 V rows take half the bytes of fp32 ones, so a bf16 stage holds
// 188 rows (180 beside the dd partials of a many-rung launch), more slots
// per staging round (Christoffel query pass 151.8 -> 148.4 us causal,
// 322.3 -> 312.6 us bidirectional, against 128).
template <typename T, int G, int RPL>
constexpr int bwd_query_cap() {
  return G >= 4 ? 72 : sizeof(T) == 4 ? kCap : RPL > 4 ? 180 : 188;
}

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* P;
  float* dP;
  float* Dvec;   // Dvec / l per (query, head)
  float* Linv;   // 1 / l per (query, head), l = sum_slots p
  float* dd_part;
  uint32_t* xq;  // packed key-pass rows (see BwdWorkspace), or null
  uint32_t* xd;
  float* wmax;   // per query-pass workgroup bound on |dS| / scale (see BwdWorkspace), or null
  const float* rope;
  int n, hq, hkv, nblk, tiles, S, n_rungs;
  int kcap;     // bwd_key: rows one stage may hold (dynamic LDS)
  int want_dd;  // bwd_query: dd requested
  int r0;       // bwd_query: first rung whose dd this launch sums (a window of RPL x ND rungs)
  float scale, scale_log2;
};

// Dot product of the lane's own head with a key chunk, summed over the lanes
// of the query (HeadSlice register order and reduce-scatter).
template <int G, int LPQ, int DC>
__device__ __forceinline__ float own_dot(const float (&a)[G][DC], const float (&b)[DC]) {
  float part[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float acc = 0.f;
#pragma unroll
    for (int x = 0; x < DC; ++x) acc = fmaf(a[h][x], b[x], acc);
    part[h] = acc;
  }
  return HeadSlice<G, LPQ>::reduce(part);
}

// RPL: dd registers per lane (0: a launch without the offset gradient).
// The LPQ / G lanes of one (query, head) hold bit-identical dot sums after
// the reduce-scatter; rung r of the launch's window [a.r0, a.r0 + RPL * ND)
// is kept by the duplicate lane u = (r - r0) % ND in register (r - r0) / ND.
// The LDS of two workgroups fits a CU, and at four heads per KV head their
// 16 waves fit the register file when a lane stays within 128 VGPRs (the
// offset-gradient registers would otherwise take it to 134): ask for that.
// Other group sizes fit (G <= 2) or do not come close (G = 8) without it.
template <int G>
constexpr int bwd_query_waves_per_eu() {
  return G == 4 ? 4 : 1;
}
template <typename T, int D, int G, int LPQ, int CAP, int BQ, int RPL>
__global__ __launch_bounds__(BQ* LPQ) __attribute__((amdgpu_waves_per_eu(bwd_query_waves_per_eu<G>())))
void bwd_query_kernel(BwdArgs a, SlotTable st) {
  constexpr int DC = D / LPQ;
  constexpr int KS = D + 4;
  constexpr int E = 16 / sizeof(T);
  constexpr int CPR = D / E;
  constexpr int NT = BQ * LPQ;
  constexpr int ND = LPQ / G;       // duplicate lanes per (query, head)
  constexpr int NWV = NT / 64;      // waves per workgroup
  constexpr int RW_DD = RPL * ND;   // rungs whose dd one launch sums
  using HS = HeadSlice<G, LPQ>;
  static_assert((ND & (ND - 1)) == 0 && NT % 64 == 0, "lane groups");
  // bf16: V rows stay the bf16 input words and dO is held as bf16 pairs, so
  // dp = dO . V takes v_dot2_f32_bf16 (exact products, fp32 sums).  V rows
  // are never interpolated: a slot that reads rows r and r - 1 forms
  // dO . V[r] and dO . V[r - 1] and lerps the two sums (the offset gradient
  // needs both anyway).  fp32 tensors: fp32 V rows, the same sums by FMA.
  constexpr bool kRawV = sizeof(T) == 2;
  constexpr int VWL = kRawV ? DC / 2 : DC;     // V words per lane
  constexpr int KSV = kRawV ? D / 2 + 4 : KS;  // words per V row (16-byte pad)
  // K and V rows of a stage, each array led by a pad row: [pad][K rows
  // 0..CAP-1][pad][V rows 0..CAP-1].  Row r - 1 of a slot (its
  // interpolation partner, or a pad row when r = 0) is then never below its
  // array, and a slot's two K rows (and its two V rows) lie at fixed byte
  // offsets from one address.
  constexpr int VOFF = (CAP + 1) * KS;  // words from the K array to the V array
  __shared__ __align__(16) float KV[(CAP + 1) * KS + (CAP + 1) * KSV];
  float* const Ks = KV + KS;
  uint32_t* const Vw = reinterpret_cast<uint32_t*>(KV + VOFF) + KSV;

  const int tid = threadIdx.x;
  const int qq = tid / LPQ;
  const int c = tid % LPQ;
  const int own = HS::own(c);
  const SeqBlock sb = lpt_seq_block(blockIdx.x, a.tiles, a.nblk);
  const int tile = sb.canon;  // index of this workgroup's dd partials
  const int seq = sb.seq;
  const int blk = sb.blk;
  const int b = seq / a.hkv, g = seq % a.hkv;
  const int n = a.n;
  const int i0 = blk * BQ;
  const int i = i0 + qq;
  const bool active = i < n;
  const int i_last = min(i0 + BQ, n) - 1;

  const T* __restrict__ Q = static_cast<const T*>(a.q);
  const T* __restrict__ K = static_cast<const T*>(a.k);
  const T* __restrict__ V = static_cast<const T*>(a.v);
  const T* __restrict__ dO = static_cast<const T*>(a.dout);

  // acc_pd = sum p dp k~, acc_p = sum p k~ ; dq~ = scale (acc_pd - Dvec acc_p)
  // Register j of a lane holds head HS::head(c, j) of the group.
  // dO: VWL words per head, bf16 pairs (bf16) or fp32 bits (fp32).
  float qv[G][DC], acc_pd[G][DC], acc_p[G][DC];
  uint32_t dow[G][VWL];
#pragma unroll
  for (int j = 0; j < G; ++j) {
    if (active) {
      const size_t off = ((size_t(b) * n + i) * a.hq + size_t(g) * G + HS::head(c, j)) * D + c * DC;
      load_vec<DC>(Q + off, qv[j]);
      if (a.rope) rotate_pairs<DC, 1>(qv[j], a.rope + size_t(i) * D, c * DC);
      load_words<VWL>(reinterpret_cast<const uint32_t*>(dO + off), dow[j]);
    } else {
#pragma unroll
      for (int x = 0; x < DC; ++x) qv[j][x] = 0.f;
#pragma unroll
      for (int x = 0; x < VWL; ++x) dow[j][x] = 0u;
    }
#pragma unroll
    for (int x = 0; x < DC; ++x) acc_pd[j][x] = acc_p[j][x] = 0.f;
  }
  const float lse2 = active ? a.lse[(size_t(b) * a.hq + size_t(g) * G + own) * n + i] * kLog2e : 0.f;
  float dvec = 0.f;  // rowsum(dO * O) of the own head, as sum_slots p dp
  // dd of the launch's rung window: X = scale p sd and Y = p (scale dp sd +
  // vd) of this lane's rungs, combined with Dvec after the slot loop.
  const bool want_dd = RPL > 0 && a.want_dd != 0;
  const int ddu = c & (ND - 1);
  float psum = 0.f;  // sum_slots p of the own head (1 up to the rounding of lse)
  // bf16 with G >= 2: max_slots |p dp| of the own head, for the bound on
  // |dS| the key pass scales its f16 weights by
  constexpr bool kBound = sizeof(T) == 2 && G >= 2;
  float umax = 0.f;
  float xacc[RPL > 0 ? RPL : 1], yacc[RPL > 0 ? RPL : 1];
#pragma unroll
  for (int r = 0; r < RPL; ++r) xacc[r] = yacc[r] = 0.f;
  // a slot whose dd this launch sums (uniform)
  auto dd_of = [&](const Slot& x) { return want_dd && unsigned(x.rung - a.r0) < unsigned(RW_DD); };

  const size_t kv_row = size_t(a.hkv) * D;
  const T* Kseq = K + size_t(b) * n * kv_row + size_t(g) * D;
  const T* Vseq = V + size_t(b) * n * kv_row + size_t(g) * D;
  const size_t ws_seq = size_t(seq) * a.S;
  // Byte offset of this lane's (query, head) entry within one slot's plane
  // of the p / dp workspace; the plane's base is uniform.
  const unsigned ws_lane = unsigned(i * G + own) * 4u;

  int s = 0;
  const int S = st.count;
  while (s < S) {
    const Slot s0 = st.s[s];  // one 16-byte scalar load per slot record
    const int lo0 = s0.lo;
    if (lo0 > i_last) break;
    // interpolated slots and dd slots read their second row i - lo - 1
    int lomax = lo0 + ((s0.frac > 0.f || dd_of(s0)) ? 1 : 0);
    int e = s + 1;
    while (e < S) {
      const Slot se = st.s[e];
      const int le = se.lo;
      if (le > i_last) break;
      const int need = max(lomax, le + ((se.frac > 0.f || dd_of(se)) ? 1 : 0));
      if (need - lo0 + BQ > CAP) break;
      lomax = need;
      ++e;
    }
    const int r0 = i0 - lomax;
    const int nrows = lomax - lo0 + BQ;

    __syncthreads();
    for (int t = tid; t < nrows * CPR; t += NT) {
      const int row = t / CPR, cc = t % CPR;
      const int pos = r0 + row;
      float kf[E];
      uint32_t vw[4];  // 16 bytes of V as they are
      if (pos >= 0 && pos < n) {
        load_vec<E>(Kseq + size_t(pos) * kv_row + cc * E, kf);
        load_words<4>(reinterpret_cast<const uint32_t*>(Vseq + size_t(pos) * kv_row + cc * E), vw);
        if (a.rope) rotate_pairs<E, 1>(kf, a.rope + size_t(pos) * D, cc * E);
      } else {
#pragma unroll
        for (int x = 0; x < E; ++x) kf[x] = 0.f;
#pragma unroll
        for (int x = 0; x < 4; ++x) vw[x] = 0u;
      }
      store_vec<E>(Ks + row * KS + cc * E, kf);
      store_words<4>(Vw + row * KSV + cc * 4, vw);
    }
    __syncthreads();

    // K and V rows r - 1 of the slot at lo = 0; a slot's rows are lo rows
    // earlier.
    const float* const lane_k = Ks + (i - r0 - 1) * KS + c * DC;
    const uint32_t* const lane_v = Vw + (i - r0 - 1) * KSV + c * VWL;
    // dO . V over the lane's dims of every head (register order)
    auto dov_dot = [&](const uint32_t (&vr)[VWL], float (&out)[G]) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int x = 0; x < VWL; ++x)
          acc = kRawV ? dot2_bf(dow[j][x], vr[x], acc) : fmaf(__uint_as_float(dow[j][x]), __uint_as_float(vr[x]), acc);
        out[j] = acc;
      }
    };
    for (int sj = s; sj < e; ++sj) {
      const Slot cur = st.s[sj];  // one 16-byte scalar load
      const int lo = cur.lo;
      // frac is +0 or positive: its bit pattern, read as an integer, decides
      // interpolation with a scalar compare.
      const int wbits = __float_as_int(cur.frac);
      const float w = __int_as_float(wbits);
      const bool interp = wbits != 0;
      const float* const kp = lane_k - lo * KS;      // K row r - 1
      const uint32_t* const vp = lane_v - lo * KSV;  // V row r - 1
      const bool dds = dd_of(cur);
      const bool two = interp || dds;  // reads rows r and r - 1
      float kt[DC], dk[DC];
      uint32_t vt[VWL], vb[VWL];
      load_vec<DC>(kp + KS, kt);
      load_words<VWL>(vp + KSV, vt);
      if (two) {
        // dK = row r - 1 minus row r: the lerp's slope and dd's factor
        float kb[DC];
        load_vec<DC>(kp, kb);
        load_words<VWL>(vp, vb);
#pragma unroll
        for (int x = 0; x < DC; ++x) dk[x] = kb[x] - kt[x];
        if (interp) {
#pragma unroll
          for (int x = 0; x < DC; ++x) kt[x] = fmaf(w, dk[x], kt[x]);
        }
      }
      float sp[G], dps[G];
#pragma unroll
      for (int j = 0; j < G; ++j) {
        float s1 = 0.f;
#pragma unroll
        for (int x = 0; x < DC; ++x) s1 = fmaf(qv[j][x], kt[x], s1);
        sp[j] = s1;
      }
      dov_dot(vt, dps);
      const float sdot = HS::reduce(sp);
      float dp = HS::reduce(dps);  // dO . V[r], the nearer row
      // Rows r and r - 1: vd = dO . (V[r - 1] - V[r]) and, for a dd slot,
      // sd = q~ . dK of the own head, fp32
      float sd = 0.f, vd = 0.f;
      if (two) {
        float vbp[G];
        dov_dot(vb, vbp);
        vd = HS::reduce(vbp) - dp;
        dp = fmaf(w, vd, dp);  // dO . lerp(V[r], V[r - 1], frac)
        if (dds) {
          float sdp[G];
#pragma unroll
          for (int j = 0; j < G; ++j) {
            float s1 = 0.f;
#pragma unroll
            for (int x = 0; x < DC; ++x) s1 = fmaf(qv[j][x], dk[x], s1);
            sdp[j] = s1;
          }
          sd = HS::reduce(sdp);
        }
      }
      // The nearer row i - lo exists when mn <= i - lo <= n - 1, mn = 1 for
      // an interpolated slot (its farther row i - lo - 1 must exist too):
      // one unsigned compare and a select, no branch.  mn comes from integer
      // arithmetic on the fraction's bits (a non-negative int), so it stays
      // in an SGPR.  Queries past n (the ragged last block) have zero q and
      // dO, so their p stays finite and is never stored.
      const int mn = min(wbits, 1);
      const bool valid = unsigned(i - lo - mn) < unsigned(n - mn);
      const float ex = __builtin_amdgcn_exp2f(sdot * a.scale_log2 - lse2);
      const float p = valid ? ex : 0.f;
      const float pdp = p * dp;
      dvec += pdp;
      psum += p;
      if constexpr (kBound) umax = fmaxf(umax, fabsf(pdp));
      if (active && HS::writer(c)) {  // p = 0 where the slot has no row for query i
        // The slot's plane bases stay scalar (global_store with an SGPR
        // base and the lane's 32-bit offset) instead of being folded into
        // per-lane 64-bit pointers.
        const size_t plane = (ws_seq + sj) * size_t(n) * G;
        float* pb = a.P + plane;
        float* db = a.dP + plane;
        asm volatile("" : "+s"(pb), "+s"(db));
        store_global_at(pb, ws_lane, p);
        store_global_at(db, ws_lane, dp);
      }
      float ph[G], pdh[G];
      HS::bcast(p, ph);
      HS::bcast(pdp, pdh);
#pragma unroll
      for (int j = 0; j < G; ++j)
#pragma unroll
        for (int x = 0; x < DC; ++x) {
          acc_pd[j][x] = fmaf(pdh[j], kt[x], acc_pd[j][x]);
          acc_p[j][x] = fmaf(ph[j], kt[x], acc_p[j][x]);
        }
      if (dds) {
        const float X = active ? a.scale * p * sd : 0.f;
        const float Y = active ? p * fmaf(a.scale * dp, sd, vd) : 0.f;
        const int rr = cur.rung - a.r0;
        const bool mine = ddu == (rr & (ND - 1));
        // The register index rr / ND is uniform: a scalar branch per
        // register (the empty asm keeps each one a branch rather than a
        // select over every register) and one select per array.
#pragma unroll
        for (int r = 0; r < RPL; ++r) {
          if (r == rr / ND) {
            asm volatile("" ::: "memory");
            xacc[r] = mine ? X : xacc[r];
            yacc[r] = mine ? Y : yacc[r];
          }
        }
      }
    }
    s = e;
  }

  // bf16 with G >= 2: this query's rows for the key pass, q~ = R(i) q and
  // dO as f16 head pairs in the key pass's LDS row layout, written once
  // here so that the key pass copies them instead of converting (and for q
  // rotating) them again in every stage that holds the row.  Register j of
  // lane c holds head own(c) ^ head(0, j), and registers 2m, 2m + 1 hold
  // the two heads of one pair: pack in register order, pick the lane's
  // register pair for each head pair, swap the halves where the even
  // register holds the odd head (v_perm with a per-lane selector).
  if constexpr (sizeof(T) == 2 && G >= 2) {
    if (active && a.xq) {
      constexpr int KC = key_chunk_h16(D, G);
      constexpr int GW = G / 2;
      static_assert(KC % DC == 0, "a lane's dims lie in one chunk");
      const int ch = (c * DC) / KC, x0 = (c * DC) % KC;
      const size_t wrow = ((size_t(seq) * n + i) * (D / KC) + ch) * (GW * KC) + x0;
      float dof[G][DC];
#pragma unroll
      for (int j = 0; j < G; ++j) words_to_floats<T, DC>(dow[j], dof[j]);
      uint32_t pq[GW][DC], pd[GW][DC];
#pragma unroll
      for (int m = 0; m < GW; ++m)
#pragma unroll
        for (int x = 0; x < DC; ++x) {
          pq[m][x] = pack_h2(qv[2 * m][x], qv[2 * m + 1][x]);
          pd[m][x] = pack_h2(dof[2 * m][x], dof[2 * m + 1][x]);
        }
#pragma unroll
      for (int hp = 0; hp < GW; ++hp) {
        // the register pair holding head pair hp, and whether its even
        // register holds the odd head
        int msel = 0;
        bool swap = false;
#pragma unroll
        for (int m = 0; m < GW; ++m) {
          const int h = HS::head(c, 2 * m);
          msel = (h >> 1) == hp ? m : msel;
          swap = (h >> 1) == hp ? (h & 1) != 0 : swap;
        }
        const uint32_t sel = swap ? 0x01000302u : 0x03020100u;  // halves swapped or kept
        uint32_t wq[DC], wd[DC];
#pragma unroll
        for (int x = 0; x < DC; ++x) {
          uint32_t q_ = pq[0][x], d_ = pd[0][x];
#pragma unroll
          for (int m = 1; m < GW; ++m) {
            q_ = msel == m ? pq[m][x] : q_;
            d_ = msel == m ? pd[m][x] : d_;
          }
          wq[x] = __builtin_amdgcn_perm(q_, q_, sel);
          wd[x] = __builtin_amdgcn_perm(d_, d_, sel);
        }
        store_words<DC>(a.xq + wrow + hp * KC, wq);
        store_words<DC>(a.xd + wrow + hp * KC, wd);
      }
    }
  }
  // p relative to l = sum p: dvn = Dvec / l is Dvec of the normalised p
  const float linv = psum > 0.f ? 1.f / psum : 0.f;
  const float dvn = dvec * linv;
  if (active && HS::writer(c)) {
    a.Dvec[(size_t(seq) * n + i) * G + own] = dvn;
    a.Linv[(size_t(seq) * n + i) * G + own] = linv;
  }
  if constexpr (kBound) {
    // |dS| / scale = |p/l (dp - dvn)| <= |p dp| / l + |dvn| (every p <= l):
    // the workgroup's maximum of that bound, for the key pass
    if (a.wmax) {
      __shared__ float wbw[NWV];
      float u = fmaf(umax, linv, fabsf(dvn));
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) u = fmaxf(u, __shfl_xor(u, m));
      if ((tid & 63) == 0) wbw[tid >> 6] = u;
      __syncthreads();
      if (tid == 0) {
        float m = wbw[0];
#pragma unroll
        for (int w_ = 1; w_ < NWV; ++w_) m = fmaxf(m, wbw[w_]);
        a.wmax[size_t(seq) * a.nblk + blk] = m;
      }
    }
  }
  if (want_dd) {
    // sum_(query, head) of Y - Dvec X per rung over the workgroup: each
    // (query, head) counts once (its duplicate lane u holds the rung), so
    // the wave sums over the lane bits above ND, then the waves are added in
    // order.  Fixed order: deterministic.  The weights are renormalised by
    // l = sum p: the rounding of the forward's lse scales every p of a query
    // by one common factor, which would otherwise enter each of the query's
    // terms (dd is a sum of many terms of both signs, so that shared error
    // does not cancel the way the terms do); with p / l the weights sum to
    // one, as the exact softmax does.
    __shared__ float ddw[NWV][RW_DD > 0 ? RW_DD : 1];
    const int lane = tid & 63, wave = tid >> 6;
#pragma unroll
    for (int r = 0; r < RPL; ++r) {
      float t = linv * fmaf(-dvn, xacc[r], yacc[r]);
#pragma unroll
      for (int m = ND; m < 64; m <<= 1) t += __shfl_xor(t, m);
      if (lane < ND) ddw[wave][r * ND + lane] = t;
    }
    __syncthreads();
    const int nr = min(a.n_rungs - a.r0, RW_DD);
    for (int r = tid; r < nr; r += NT) {
      float t = 0.f;
#pragma unroll
      for (int w_ = 0; w_ < NWV; ++w_) t += ddw[w_][r];
      a.dd_part[size_t(a.r0 + r) * a.tiles + tile] = t;
    }
  }
  // dq~ = scale / l (sum p dp k~ - dvn sum p k~)
  float dvh[G], slh[G];
  HS::bcast(dvn, dvh);
  HS::bcast(a.scale * linv, slh);
  if (active) {
    T* dQ = static_cast<T*>(a.dq);
#pragma unroll
    for (int j = 0; j < G; ++j) {
      float dq[DC];
#pragma unroll
      for (int x = 0; x < DC; ++x) dq[x] = slh[j] * fmaf(-dvh[j], acc_p[j][x], acc_pd[j][x]);
      if (a.rope) rotate_pairs<DC, -1>(dq, a.rope + size_t(i) * D, c * DC);
      store_vec<DC>(dQ + ((size_t(b) * n + i) * a.hq + size_t(g) * G + HS::head(c, j)) * D + c * DC, dq);
    }
  }
}

// Key-centric pass.  For key j and slot s (row pair i-lo, i-lo-1 of query
// i): tap 0 is query j+lo (weight 1-frac), tap 1 is query j+lo+1 (weight
// frac; only for an interpolated slot).  dS = scale p (dp - Dvec) is formed
// here from the stored p, dp and Dvec.
//
// One workgroup per (sequence, block of KB keys, chunk of KC dims); one key
// per lane.  The query rows a stage of slots needs, [j0 + lo_first,
// j0 + KB - 1 + lo_last + 1], are staged once into LDS as raw Q and dO
// elements of the chunk for all G heads, so each row read from L2 serves
// every (slot, tap) of the stage.  p, dp and Dvec of the next (slot, tap)
// are loaded one step ahead.

// Keys per workgroup: 128 (two waves) when a staged row (Q and dO of the
// chunk for all heads) is at most 256 bytes, else 64; a stage holds the
// block plus 48 rows of slot spread.
constexpr int key_block(int esize, int G, int D) {
  return 2 * G * key_chunk(D) * esize <= 256 ? 128 : 64;
}
constexpr int key_cap(int kb) { return kb + 48; }

struct ReduceArgs {
  const float* dd_part;
  float* dd;
  float* dtheta;
  int blocks, n_rungs;
  double alpha;
  float base[SFA_MAX_OFFSETS];
};

// dd and dtheta from the query pass's partials, by one workgroup of NT
// threads.  The partials (one per query-pass workgroup) are stored
// rung-major ([rung][block]), so wave w reduces rungs w, w + NT/64, ... with
// coalesced loads: lane l adds the partials of blocks l, l+64, ... in block
// order, then the wave adds its 64 lanes in a fixed shuffle tree, all in
// double (a dd_k is a sum over every query and head of the batch, often a
// near cancellation).  The order does not depend on NT or on timing.  sdd:
// n_rungs doubles of LDS.
__device__ __forceinline__ void reduce_body(const ReduceArgs& a, double* sdd, int nt) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  for (int r = wave; r < a.n_rungs; r += nt / 64) {
    double acc = 0.0;
    const float* row = a.dd_part + size_t(r) * a.blocks;
    int blk = lane;
    for (; blk + 7 * 64 < a.blocks; blk += 8 * 64) {
      float x[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) x[u] = row[blk + u * 64];
#pragma unroll
      for (int u = 0; u < 8; ++u) acc += double(x[u]);
    }
    for (; blk < a.blocks; blk += 64) acc += double(row[blk]);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) acc += __shfl_xor(acc, m);
    if (lane == 0) {
      sdd[r] = acc;
      if (a.dd) a.dd[r] = float(acc);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0 && a.dtheta) {
    double da = 0.0;
    for (int r = 0; r < a.n_rungs; ++r) da += double(a.base[r]) * sdd[r];
    a.dtheta[0] = float((a.alpha - 0.5) * (1.5 - a.alpha) * da);
  }
}

// The reduction as a kernel of its own (the float32 backward and the empty
// problem), one workgroup of 16 waves.
constexpr int kReduceThreads = 1024;

__global__ __launch_bounds__(kReduceThreads) void bwd_reduce_kernel(ReduceArgs a) {
  __shared__ double sdd[SFA_MAX_OFFSETS];
  reduce_body(a, sdd, kReduceThreads);
}

// bf16 key pass: workgroups of 256 keys (four waves) of two kinds in one
// launch, dK (staging q~) and dV (staging dO).  Words per staged row: the
// chunk of every head as f16 head pairs, plus a 4-word pad against bank
// conflicts.  A stage stages the block's rows plus the slots' spread, so a
// longer block re-stages fewer rows per key: against 128 keys (two waves,
// the same 16 waves per CU) the page-1 key pass went 83.1 -> 80.1 us and the
// Christoffel one 122.3 -> 102.0 us; 512 keys were slower than 256 on both.
constexpr int kKeyBlockH16 = 256;
// Words per staged row: the chunk of every head as f16 head pairs (G >= 2,
// one half of the pass per workgroup), or with one head per KV head the fp32
// chunks of q~ and dO together (both halves in one workgroup); plus a 4-word
// pad.
constexpr int key_half_row_words(int G, int D) {
  return G == 1 ? 2 * key_chunk_h16(D, G) + 4 : key_chunk_h16(D, G) * ((G + 1) / 2) + 4;
}

// The (slot, tap) steps of the bf16 key pass in order, built on the host
// from the slot table and passed by value like it (the same size): per step
// the row delta min(lo, n) + tap, and the tap weight (1 - frac for the
// nearer row, frac for the farther one, 1 for an integer slot) with its sign
// bit, free since the weight is positive, set on a slot's first step.  lo of
// the first and last slot bound the rows whose dS bounds scale the dK
// weights.
struct StepTable {
  int32_t count;  // steps
  int32_t lo_first, lo_last;
  int32_t pad_;
  uint2 rec[2 * SFA_MAX_SLOTS];
};
static_assert(sizeof(StepTable) == sizeof(SlotTable), "steps travel like the slots");

inline StepTable make_step_table(const SlotTable& t, int n) {
  StepTable st{};
  for (int x = 0; x < t.count; ++x) {
    const int d0 = t.s[x].lo < n ? t.s[x].lo : n;
    const float fr = t.s[x].frac;
    float w0 = 1.f;
    if (fr > 0.f) w0 = 1.f - fr;
    uint32_t b0, b1;
    std::memcpy(&b0, &w0, 4);
    std::memcpy(&b1, &fr, 4);
    st.rec[st.count++] = make_uint2(uint32_t(d0), b0 | 0x80000000u);
    if (fr > 0.f) st.rec[st.count++] = make_uint2(uint32_t(d0 + 1), b1);
  }
  st.lo_first = t.count > 0 ? t.s[0].lo : 0;
  st.lo_last = t.count > 0 ? t.s[t.count - 1].lo : 0;
  return st;
}

// Rows per stage of a bf16 key-pass half.  As many as let 16 waves per CU
// share the 160 KiB of LDS, but at least the block plus 12 rows (a window
// of 10 and the interpolation tap in one stage; with offsets 8 apart, as in
// page 3's layer, two offsets per stage: a capacity of the block plus 7
// measured 163 against 160 us causal and 433 against 349 us bidirectional)
// and at most the block plus 64.
inline int key_half_cap(int G, int D) {
  constexpr int kb = kKeyBlockH16, nw = kb / 64;
  const int budget = 163840 * nw / 16;
  int cap = budget / (4 * key_half_row_words(G, D));
  if (cap < kb + 12) cap = kb + 12;
  if (cap > kb + 64) cap = kb + 64;
  return cap;
}

template <typename T, int D, int G>
__global__ __launch_bounds__(key_block(sizeof(T), G, D)) void bwd_key_kernel(BwdArgs a, SlotTable st) {
  constexpr int KB = key_block(sizeof(T), G, D);
  constexpr int KCAP = key_cap(KB);
  constexpr int KC = key_chunk(D);
  constexpr int NCH = D / KC;
  constexpr int HW = KC * int(sizeof(T)) / 4;  // 32-bit words per head chunk
  constexpr int RW = 2 * G * HW + 4;           // words per staged row (Q, dO, pad)
  constexpr int CH16 = KC * int(sizeof(T)) / 16;  // 16-byte pieces per head chunk
  constexpr int PPR = 2 * G * CH16;               // 16-byte pieces per row
  static_assert(KC * sizeof(T) % 16 == 0, "16-byte pieces");
  __shared__ __align__(16) uint32_t Ws[KCAP * RW];

  const int tid = threadIdx.x;
  const int tile = xcd_tile(blockIdx.x, a.tiles);
  const int c = tile % NCH;
  const int rest = tile / NCH;
  const int seq = rest / a.nblk;
  const int blk = rest % a.nblk;
  const int b = seq / a.hkv, g = seq % a.hkv;
  const int n = a.n;
  const int j0 = blk * KB;
  const int j = j0 + tid;
  const bool activej = j < n;

  const T* __restrict__ Q = static_cast<const T*>(a.q);
  const T* __restrict__ dO = static_cast<const T*>(a.dout);
  const size_t ws_seq = size_t(seq) * a.S;
  const size_t kv_off = (size_t(b) * n + j) * size_t(a.hkv) * D + size_t(g) * D + c * KC;

  float dk[KC], dv[KC];
#pragma unroll
  for (int x = 0; x < KC; ++x) dk[x] = dv[x] = 0.f;

  const int S = st.count;
  int s = 0;
  while (s < S) {
    const int lo0 = st.s[s].lo;
    if (j0 + lo0 > n - 1) break;  // no query at this distance for any key of the block
    int lomax = lo0;
    int e = s;
    while (e < S) {
      const int le = st.s[e].lo;
      if (j0 + le > n - 1 || le - lo0 + KB + 1 > KCAP) break;
      lomax = le;
      ++e;
    }
    const int r0 = j0 + lo0;                              // query row of LDS row 0
    const int nrows = min(lomax - lo0 + KB + 1, n - r0);  // rows past n are never read

    __syncthreads();
    for (int t = tid; t < nrows * PPR; t += KB) {
      const int row = t / PPR, piece = t % PPR;
      const int which = piece / (G * CH16);  // 0: Q, 1: dO
      const int h = (piece / CH16) % G;
      const int part = piece % CH16;
      uint4 x = make_uint4(0, 0, 0, 0);  // rows before the sequence (negative offsets) stay zero
      if (r0 + row >= 0) {
        const T* src = (which ? dO : Q) + ((size_t(b) * n + r0 + row) * a.hq + size_t(g) * G + h) * D + c * KC +
                       part * (16 / int(sizeof(T)));
        x = *reinterpret_cast<const uint4*>(src);
      }
      *reinterpret_cast<uint4*>(Ws + row * RW + (which * G + h) * HW + part * 4) = x;
    }
    __syncthreads();

    // (slot, tap) steps of this stage, with the workspace loads of the next
    // step issued before the current one is consumed.
    auto step_valid = [&](int sj, int tap) {
      const float w = st.s[sj].frac;
      const int i = j + st.s[sj].lo + tap;
      return activej && i >= 0 && i < n && (tap == 1 || j > 0 || w == 0.f);
    };
    // p is loaded as p / l (times the stored 1/l of its query and head)
    auto load_step = [&](int sj, int tap, float (&pg)[G], float (&dpg)[G], float (&dvg)[G]) {
      if (step_valid(sj, tap)) {
        const int i = j + st.s[sj].lo + tap;
        const size_t widx = ((ws_seq + sj) * n + i) * G;
        float lg[G];
        load_vec<G>(a.P + widx, pg);
        load_vec<G>(a.dP + widx, dpg);
        load_vec<G>(a.Dvec + (size_t(seq) * n + i) * G, dvg);
        load_vec<G>(a.Linv + (size_t(seq) * n + i) * G, lg);
#pragma unroll
        for (int h = 0; h < G; ++h) pg[h] *= lg[h];
      } else {
#pragma unroll
        for (int h = 0; h < G; ++h) pg[h] = dpg[h] = dvg[h] = 0.f;
      }
    };
    auto taps_of = [&](int sj) { return st.s[sj].frac > 0.f ? 2 : 1; };

    float pg[G], dpg[G], dvg[G];
    load_step(s, 0, pg, dpg, dvg);
    int sj = s, tap = 0;
    while (sj < e) {
      int nsj = sj, ntap = tap + 1;
      if (ntap >= taps_of(sj)) {
        ++nsj;
        ntap = 0;
      }
      float pn[G], dpn[G], dvn[G];
      if (nsj < e) load_step(nsj, ntap, pn, dpn, dvn);

      const int lo = st.s[sj].lo;
      const float w = st.s[sj].frac;
      const int delta = lo + tap;
      const float wt = tap ? w : 1.f - w;
      const bool valid = step_valid(sj, tap);
      float yk[KC], yv[KC];
#pragma unroll
      for (int x = 0; x < KC; ++x) yk[x] = yv[x] = 0.f;
      if (valid) {
        const uint32_t* rowp = Ws + (j + delta - r0) * RW;
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float dsh = a.scale * pg[h] * (dpg[h] - dvg[h]);
          float qh[KC], oh[KC];
          load_vec<KC>(reinterpret_cast<const T*>(rowp + h * HW), qh);
          load_vec<KC>(reinterpret_cast<const T*>(rowp + (G + h) * HW), oh);
#pragma unroll
          for (int x = 0; x < KC; ++x) {
            yk[x] = fmaf(dsh, qh[x], yk[x]);
            yv[x] = fmaf(pg[h], oh[x], yv[x]);
          }
        }
        if (a.rope) {
          // R(delta) into key j's frame; a negative (future) offset rotates
          // by R(|delta|)^T.  |delta| = |i - j| < n for a valid step.
          if (delta >= 0)
            rotate_pairs<KC, 1>(yk, a.rope + size_t(delta) * D, c * KC);
          else
            rotate_pairs<KC, -1>(yk, a.rope + size_t(-delta) * D, c * KC);
        }
#pragma unroll
        for (int x = 0; x < KC; ++x) {
          dk[x] = fmaf(wt, yk[x], dk[x]);
          dv[x] = fmaf(wt, yv[x], dv[x]);
        }
      }
      if (nsj < e) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
          pg[h] = pn[h];
          dpg[h] = dpn[h];
          dvg[h] = dvn[h];
        }
      }
      sj = nsj;
      tap = ntap;
    }
    s = e;
  }
  if (activej) {
    store_vec<KC>(static_cast<T*>(a.dk) + kv_off, dk);
    store_vec<KC>(static_cast<T*>(a.dv) + kv_off, dv);
  }
}

// bf16 tensors: the key pass with f16 operands, split into two halves that
// each stage half of a query row (one launch, bwd_key_h16_kernel below, runs
// both).  PART 0 (dK) stages q~ = R(i) q of the
// chunk (rotated while staging) and gathers yk~ = sum_h dS_h q~_h; dK~ =
// sum w yk~ is rotated back once, dK = R(j)^T dK~ (the relative rotation
// R(i - j) = R(j)^T R(i) never has to be formed per step).  PART 1 (dV)
// stages dO and gathers yv = sum_h p_h dO_h: dV += w yv.  A staged row holds the chunk of every head as f16 with the
// heads interleaved in pairs (word [hp][x] = (head 2hp, head 2hp+1) of dim
// x), so each head sum is one v_dot2_f32_f16 per head pair and dim,
// accumulated in fp32; dS and p enter as f16 pairs.  Half a row per
// workgroup halves the LDS and registers per wave, so four waves share a
// SIMD.  With one head per KV head (G = 1) a pair would leave half of every
// f16 word empty, so there the staged words hold the fp32 rows and the
// weights stay fp32 (one FMA per dim and step instead of a dot2 doing one
// useful MAC), and PART 2 does both halves in one workgroup: a step is then
// 32 FMAs (dK and dV) for one set of per-step bookkeeping (step record,
// weight loads, ring address), which is scalar work that otherwise bounds
// the pass (more SALU than VALU instructions per wave with the halves
// apart).
template <int D, int G, int PART>
__device__ __forceinline__ void key_half_body(const BwdArgs& a, const StepTable& st, const int tile) {
  constexpr int KB = kKeyBlockH16;
  constexpr int KC = key_chunk_h16(D, G);
  constexpr int NCH = D / KC;
  constexpr int GW = (G + 1) / 2;  // head pairs
  constexpr int RW = key_half_row_words(G, D);
  constexpr int XH = KC / 8;       // 8-dim pieces per head chunk
  constexpr bool BOTH = PART == 2;  // dK and dV in one workgroup (G = 1)
  static_assert(!BOTH || G == 1, "both halves only with one head per KV head");
  constexpr int PPR = (BOTH ? 2 : GW) * XH;  // staging pieces per row
  // steps of weight loads in flight (2 and 4 were measured slower: the key
  // pass is not bound by their latency)
  constexpr int PF = 1;
  static_assert(KC % 8 == 0 && KB % PPR == 0, "8-dim pieces, whole rows per pass");
  // Dynamic LDS: a.kcap staged rows of RW words.
  extern __shared__ __align__(16) uint32_t key_smem[];
  uint32_t* Ws = key_smem;

  const int tid = threadIdx.x;
  const int c = tile % NCH;
  const int rest = tile / NCH;
  const int seq = rest / a.nblk;
  const int blk = rest % a.nblk;
  const int b = seq / a.hkv, g = seq % a.hkv;
  const int n = a.n;
  const int j0 = blk * KB;
  const int j = j0 + tid;
  const bool activej = j < n;
  const bool rope = PART != 1 && a.rope != nullptr;

  const bf16_t* __restrict__ X = static_cast<const bf16_t*>(PART == 1 ? a.dout : a.q);
  const size_t kv_off = (size_t(b) * n + j) * size_t(a.hkv) * D + size_t(g) * D + c * KC;

  float acc[KC], accv[BOTH ? KC : 1];  // dK~ (or dV), and dV for BOTH

  // dK with f16 weights: dS = scale p (dp - Dvec) scales with dO and V and
  // can fall below f16's normal range (2^-14) while both are well inside
  // it, losing the weights' precision.  The weights enter scaled by 2^e,
  // e chosen so that the largest bound on |dS| over the query-pass
  // workgroups holding this block's rows [j0 + lo_first, j0 + KB + lo_last]
  // maps to [2^13, 2^14), and the sum is scaled back by 2^-e before the
  // store (both exact).  Each wave takes the maximum itself (no barrier);
  // the waves agree, and each scales back its own keys either way.
  float kscale = a.scale, kunscale = 1.f;
  if constexpr (PART == 0 && !BOTH) {
    if (a.wmax && st.count > 0) {
      constexpr int BQQ = bwd_bq<G>();
      const int nq = (n + BQQ - 1) / BQQ;
      const int ilo = max(j0 + max(st.lo_first, -n), 0);
      const int ihi = min(j0 + KB + min(st.lo_last, n), n - 1);
      float u = 0.f;
      if (ilo <= ihi) {
        const float* wm = a.wmax + size_t(seq) * nq;
        for (int t = ilo / BQQ + (tid & 63); t <= ihi / BQQ; t += 64) u = fmaxf(u, wm[t]);
      }
#pragma unroll
      for (int m = 1; m < 64; m <<= 1) u = fmaxf(u, __shfl_xor(u, m));
      const float w = a.scale * u;
      if (w > 0.f && w <= 3.4e38f) {
        int ex;
        (void)frexpf(w, &ex);  // w < 2^ex
        const int e = min(max(14 - ex, -120), 120);
        kscale = ldexpf(a.scale, e);
        kunscale = ldexpf(1.f, -e);
      }
    }
  }
#pragma unroll
  for (int x = 0; x < KC; ++x) acc[x] = 0.f;
#pragma unroll
  for (int x = 0; x < (BOTH ? KC : 1); ++x) accv[x] = 0.f;

  // The step loop reads one record of the step table per step (a scalar
  // load issued a step ahead): no per-step cursor branches, and the p and dp
  // planes move to the next slot's by a scalar select on a slot's first
  // step (page-1 key pass 78.9 -> 73.2 us against a cursor over the slots).
  const int nsteps = st.count;
  auto first_of_slot = [&](int t) { return (st.rec[t].y >> 31) != 0u; };

  // p and 1/l (and for dK dp and Dvec / l) of one step, loaded without a
  // branch: the row is clamped to n - 1, and every clamped row is one the
  // query pass wrote (a slot is only reached while j0 + lo <= n - 1).  A step
  // past the end reloads the last step's rows; masked steps get zero weights
  // in convert().  raw: p, 1/l (dV); p, dp, Dvec / l, 1/l (dK).
  constexpr int NR = PART == 1 ? 2 : 4;
  constexpr int RL = NR - 1;  // the 1/l entry
  constexpr int NWT = BOTH ? 2 : GW;  // weight words per step
  // Scalar bases of this sequence's p, dp and Dvec; a slot's plane is a
  // scalar byte offset from them, the row a 32-bit lane offset.
  const float* const Pseq = uniform_ptr(a.P + size_t(seq) * a.S * n * G);
  const float* const dPseq = uniform_ptr(a.dP + size_t(seq) * a.S * n * G);
  const float* const Dseq = uniform_ptr(a.Dvec + size_t(seq) * n * G);
  const float* const Lseq = uniform_ptr(a.Linv + size_t(seq) * n * G);
  const unsigned plane_b = unsigned(n) * unsigned(G * 4);
  // The loader: the step whose loads are queued next, the byte offset of its
  // slot's plane (one plane before slot 0 until step 0 moves it there; kept
  // at the last slot once past the end) and its record.
  int fstep = 0;
  unsigned fplane = 0u - plane_b;
  uint2 frec = make_uint2(0u, 0u);
  if (nsteps > 0) frec = st.rec[0];
  // A queue entry: the loads of one step, its weight factor (the tap weight,
  // or 0 for a masked step), its index (nsteps past the end) and its row
  // delta lo + tap.
  struct QE {
    float raw[NR][G];
    float ws;
    int step, delta;
  };
  // The loads share the lane's 32-bit byte offset i * G * 4 from uniform
  // bases (the slot's planes of p and dp, and Dvec), so the address
  // arithmetic is scalar except for that offset.
  auto load_step = [&](QE& q) {
    const int delta = int(frec.x);
    const uint32_t wb = frec.y;
    const bool live = fstep < nsteps;
    fplane += live && (wb >> 31) ? plane_b : 0u;
    const int i = min(max(j + delta, 0), n - 1);
    const unsigned ioff = unsigned(i) * unsigned(G * 4);
    load_global_at<G>(Pseq, fplane + ioff, q.raw[0]);
    if constexpr (PART != 1) {
      load_global_at<G>(dPseq, fplane + ioff, q.raw[1]);
      load_global_at<G>(Dseq, ioff, q.raw[2]);
    }
    load_global_at<G>(Lseq, ioff, q.raw[RL]);
    const bool valid = live && unsigned(j + delta) < unsigned(n);
    q.ws = valid ? __uint_as_float(wb & 0x7fffffffu) : 0.f;
    q.step = fstep;
    q.delta = delta;
    fstep += live ? 1 : 0;
    frec = st.rec[min(fstep, nsteps - 1)];  // the next record, a step ahead
  };
  // f16 weight pairs of a queued step (G = 1: one fp32 weight): ws dS, dS =
  // p/l (dp - Dvec/l), for dK, ws p/l for dV.  Every loaded value is finite
  // (a clamped row the query pass wrote), so a masked step's ws = 0 gives 0.
  auto convert = [&](const QE& q, uint32_t (&wts)[NWT]) {
    if constexpr (BOTH) {
      const float p = q.ws * q.raw[0][0] * q.raw[RL][0];
      wts[0] = __float_as_uint(a.scale * p * (q.raw[1][0] - q.raw[2][0]));
      wts[1] = __float_as_uint(p);
    } else {
      const float ws = PART == 0 ? kscale * q.ws : q.ws;
#pragma unroll
      for (int hp = 0; hp < GW; ++hp) {
        const int h0 = 2 * hp, h1 = 2 * hp + 1 < G ? 2 * hp + 1 : 2 * hp;
        float w0 = q.raw[0][h0] * q.raw[RL][h0], w1 = 2 * hp + 1 < G ? q.raw[0][h1] * q.raw[RL][h1] : 0.f;
        if constexpr (PART == 0) {
          w0 = ws * w0 * (q.raw[1][h0] - q.raw[2][h0]);
          w1 = ws * w1 * (q.raw[1][h1] - q.raw[2][h1]);
        } else {
          w0 *= ws;
          w1 *= ws;
        }
        wts[hp] = G == 1 ? __float_as_uint(w0) : pack_h2(w0, w1);
      }
    }
  };

  // Software pipeline along the steps, straight across stage boundaries:
  // wts holds the weights of the step being computed and the queue the loads
  // of the PF steps after it.  The end of each step converts the queue's
  // head into the next weights, shifts the queue and loads the step PF
  // ahead, so every load has PF steps to arrive.
  uint32_t wts[NWT] = {};
  int wstep = nsteps, wdelta = 0;  // step being computed and its row delta
  QE que[PF];
  if (nsteps > 0) {
    load_step(que[0]);
    convert(que[0], wts);
    wstep = que[0].step;
    wdelta = que[0].delta;
#pragma unroll
    for (int k = 0; k < PF; ++k) load_step(que[k]);
  }
  // The staged rows form a ring in LDS: query j0 + q sits in slot
  // (q - q0) mod kcap, q0 the first stage's first row.  Stages run in
  // increasing offset order and each spans at most kcap rows, so rows that an
  // earlier stage staged and the new stage still needs ([lo0, have_hi]) are
  // intact, and only the rows above have_hi are staged (consecutive rungs
  // share most of their rows).
  const int kcap = a.kcap;
  // Byte offset of ring slot tid.  Opaque to the compiler, which would
  // otherwise fold it back into (tid + soff) * RW * 4 per step, a
  // quarter-rate integer multiply.
  unsigned tid_b = unsigned(tid * RW * 4);
  asm volatile("" : "+v"(tid_b));
  int q0 = 0, have_hi = 0;
  bool first_stage = true;
  int ts = 0;  // the stage's first step (a slot's first)
  while (ts < nsteps) {
    const int lo0 = int(st.rec[ts].x);  // min(lo, n) of the stage's first slot
    if (j0 + lo0 > n - 1) break;
    int lomax = lo0;
    int te = ts;  // a stage holds whole slots: steps [ts, te)
    while (te < nsteps) {
      const int le = int(st.rec[te].x);
      if (j0 + le > n - 1 || le - lo0 + KB + 1 > kcap) break;
      lomax = le;
      te += te + 1 < nsteps && !first_of_slot(te + 1) ? 2 : 1;
    }
    const int r0 = j0 + lo0;
    const int nrows = min(lomax - lo0 + KB + 1, n - r0);
    const int hi = lo0 + nrows - 1;  // last row of the stage, relative to j0
    if (first_stage) {
      q0 = lo0;
      have_hi = lo0 - 1;
      first_stage = false;
    }
    const int base = (lo0 - q0) % kcap;    // ring slot of row lo0 (lo0 >= q0)
    const int fnew = max(lo0, have_hi + 1);  // first row not staged yet
    const int nnew = hi - fnew + 1;

    __syncthreads();

    // Thread t always stages piece t % PPR of a row, rows t / PPR,
    // t / PPR + KB / PPR, ...  With G >= 2 the query pass has written the
    // rows already in this layout (f16 head pairs, q rotated by its own
    // position), so a piece is a copy of 8 words.
    if constexpr (G >= 2) {
      constexpr int SB = 4;
      constexpr int RSTEP = KB / PPR;
      const int pc = tid % PPR;
      const int hp = pc / XH;
      const int xh = pc % XH;
      const uint32_t* __restrict__ XP = PART == 0 ? a.xq : a.xd;
      const int rn = j0 + fnew;  // query of the first new row
      // word offset of piece (hp, xh) of chunk c within a packed row
      const uint32_t* src0 = XP + size_t(seq) * n * (D * GW) + (c * GW + hp) * KC + xh * 8;
      uint32_t* dst0 = Ws + hp * KC + xh * 8;
      for (int row0 = tid / PPR; row0 < nnew; row0 += SB * RSTEP) {
        uint4 u0[SB], u1[SB];
#pragma unroll
        for (int u = 0; u < SB; ++u) {
          const int row = row0 + u * RSTEP;
          u0[u] = u1[u] = make_uint4(0, 0, 0, 0);
          // rows before the sequence (negative offsets) are staged as zeros;
          // masked steps read ring slot 0 with zero weights
          if (row < nnew && rn + row >= 0) {
            const uint32_t* src = src0 + int64_t(rn + row) * (D * GW);
            u0[u] = *reinterpret_cast<const uint4*>(src);
            u1[u] = *reinterpret_cast<const uint4*>(src + 4);
          }
        }
#pragma unroll
        for (int u = 0; u < SB; ++u) {
          const int row = row0 + u * RSTEP;
          if (row < nnew) {
            int slot = fnew - lo0 + row + base;  // < 2 kcap
            slot = slot >= kcap ? slot - kcap : slot;
            uint32_t* dst = dst0 + slot * RW;
            *reinterpret_cast<uint4*>(dst) = u0[u];
            *reinterpret_cast<uint4*>(dst + 4) = u1[u];
          }
        }
      }
    } else {
      // G = 1: fp32 words, converted here; dK rows are rotated by their own
      // position, R(i) q, on the way.  Batches of SB pieces: all their
      // global loads are issued before the first conversion.
      constexpr int SB = PART == 1 ? 4 : 2;  // dK also holds rotary rows
      constexpr int RSTEP = KB / PPR;
      const int pc = tid % PPR;
      const int hp = pc / XH;  // head pair; with BOTH: 0 stages q~, 1 dO
      const int xh = pc % XH;
      const bool pair = !BOTH && 2 * hp + 1 < G;
      const bool rot = rope && !(BOTH && hp == 1);  // q~ rows are rotated, dO rows not
      const bf16_t* __restrict__ Xs = BOTH ? static_cast<const bf16_t*>(hp ? a.dout : a.q) : X;
      const size_t rstride = size_t(a.hq) * D;
      // addresses from signed row indices: rows < 0 with negative offsets
      const int rn = j0 + fnew;                   // query of the first new row
      const int64_t grow0 = int64_t(b) * n + rn;  // its global row
      const size_t col = (size_t(g) * G + (BOTH ? 0 : 2 * hp)) * D + c * KC + xh * 8;
      uint32_t* dst0 = Ws + hp * KC + xh * 8;
      for (int row0 = tid / PPR; row0 < nnew; row0 += SB * RSTEP) {
        uint4 u0[SB], u1[SB];
        float4 ra[SB], rb[SB];
#pragma unroll
        for (int u = 0; u < SB; ++u) {
          const int row = row0 + u * RSTEP;
          u0[u] = u1[u] = make_uint4(0, 0, 0, 0);
          ra[u] = rb[u] = make_float4(1.f, 0.f, 1.f, 0.f);
          // rows before the sequence (negative offsets) are staged as zeros;
          // masked steps read ring slot 0 with zero weights
          if (row < nnew && rn + row >= 0) {
            const bf16_t* src = Xs + size_t(grow0 + row) * rstride + col;
            u0[u] = *reinterpret_cast<const uint4*>(src);
            if (pair) u1[u] = *reinterpret_cast<const uint4*>(src + D);
            if (rot) {
              const float* rp = a.rope + size_t(rn + row) * D + c * KC + xh * 8;
              ra[u] = *reinterpret_cast<const float4*>(rp);
              rb[u] = *reinterpret_cast<const float4*>(rp + 4);
            }
          }
        }
#pragma unroll
        for (int u = 0; u < SB; ++u) {
          const int row = row0 + u * RSTEP;
          if (row < nnew) {
            const uint32_t e0[4] = {u0[u].x, u0[u].y, u0[u].z, u0[u].w};
            const uint32_t e1[4] = {u1[u].x, u1[u].y, u1[u].z, u1[u].w};
            const float cs[8] = {ra[u].x, ra[u].y, ra[u].z, ra[u].w, rb[u].x, rb[u].y, rb[u].z, rb[u].w};
            uint32_t wv[8];
#pragma unroll
            for (int x = 0; x < 4; ++x) {
              // dims 2x, 2x + 1 of both heads: one rotation pair each
              float a0 = bf16_lo(e0[x]), b0 = bf16_hi(e0[x]);
              float a1 = bf16_lo(e1[x]), b1 = bf16_hi(e1[x]);
              if (PART != 1) {  // rows that are not rotated carry the identity (cos 1, sin 0)
                const float c_ = cs[2 * x], s_ = cs[2 * x + 1];
                const float ra0 = a0 * c_ - b0 * s_, rb0 = a0 * s_ + b0 * c_;
                const float ra1 = a1 * c_ - b1 * s_, rb1 = a1 * s_ + b1 * c_;
                a0 = ra0; b0 = rb0; a1 = ra1; b1 = rb1;
              }
              if constexpr (G == 1) {
                wv[2 * x] = __float_as_uint(a0);
                wv[2 * x + 1] = __float_as_uint(b0);
              } else {
                wv[2 * x] = pack_h2(a0, a1);
                wv[2 * x + 1] = pack_h2(b0, b1);
              }
            }
            int slot = fnew - lo0 + row + base;  // < 2 kcap
            slot = slot >= kcap ? slot - kcap : slot;
            uint32_t* dst = dst0 + slot * RW;
            *reinterpret_cast<uint4*>(dst) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
            *reinterpret_cast<uint4*>(dst + 4) = make_uint4(wv[4], wv[5], wv[6], wv[7]);
          }
        }
      }
    }
    __syncthreads();
    have_hi = max(have_hi, hi);

    // every step of the stage
    while (wstep < te) {
      {
        // The next record's scalar load lands here, before the row reads:
        // with it still in flight every wait on the row reads would have to
        // drain all LDS reads.
        asm volatile("" ::"s"(frec.x), "s"(frec.y));
        const int delta = wdelta;
        // Query j + delta; the query pass stored p = 0 where the slot has no
        // row for it.  Masked steps read ring slot 0 with zero weights.
        // The tap weight (1 - frac or frac) is already in the step's
        // weights.  One straight-line body keeps the registers put.
        // Ring slot of query j + delta: tid + soff (soff uniform), wrapped
        // once past kcap; as a byte offset, the lane's tid * RW * 4 plus a
        // scalar term, minus the ring size where tid >= kcap - soff.
        const bool valid = unsigned(j + delta) < unsigned(n);
        const int soff = delta - lo0 + base;  // j + delta - r0 = tid + delta - lo0
        const unsigned wrap = tid >= kcap - soff ? unsigned(kcap * RW * 4) : 0u;
        const unsigned roff = tid_b + unsigned(soff * RW * 4) - wrap;
        const uint32_t* rowp = reinterpret_cast<const uint32_t*>(
            reinterpret_cast<const char*>(Ws) + (valid ? roff : 0u));
        if constexpr (BOTH) {
          // dK~ += (wt dS) q~ and dV += (wt p) dO
          uint32_t xq[KC], xd[KC];
          load_words<KC>(rowp, xq);
          load_words<KC>(rowp + KC, xd);
          const float wk = __uint_as_float(wts[0]), wv = __uint_as_float(wts[1]);
#pragma unroll
          for (int x = 0; x < KC; ++x) {
            acc[x] = fmaf(wk, __uint_as_float(xq[x]), acc[x]);
            accv[x] = fmaf(wv, __uint_as_float(xd[x]), accv[x]);
          }
        } else if constexpr (G == 1) {
          // acc += (wt w0) x
          uint32_t xw[KC];
          load_words<KC>(rowp, xw);
          const float w0 = __uint_as_float(wts[0]);
#pragma unroll
          for (int x = 0; x < KC; ++x) acc[x] = fmaf(w0, __uint_as_float(xw[x]), acc[x]);
        } else {
          // acc += sum over head pairs of dot2((wt w_2hp, wt w_2hp+1), x)
          uint32_t xw[KC];
#pragma unroll
          for (int hp = 0; hp < GW; ++hp) {
            load_words<KC>(rowp + hp * KC, xw);
#pragma unroll
            for (int x = 0; x < KC; ++x) acc[x] = dot2_h(wts[hp], xw[x], acc[x]);
          }
        }

        // weights of the next step, then the loads of the step PF ahead.
        // The barrier keeps the conversion, which waits for the queued
        // loads, after this step's row reads and dot products: hoisted above
        // them it made every step wait for its weights before reading its
        // rows (page-1 key pass 84.2 against 79 us).
        __builtin_amdgcn_sched_barrier(0);
        convert(que[0], wts);
        wstep = que[0].step;
        wdelta = que[0].delta;
#pragma unroll
        for (int k = 0; k + 1 < PF; ++k) que[k] = que[k + 1];
        __builtin_amdgcn_sched_barrier(0);
        load_step(que[PF - 1]);
      }
    }
    ts = te;
  }
  if (activej) {
    if constexpr (PART == 0 && !BOTH) {
#pragma unroll
      for (int x = 0; x < KC; ++x) acc[x] *= kunscale;
    }
    if (rope) rotate_pairs<KC, -1>(acc, a.rope + size_t(j) * D, c * KC);  // dK = R(j)^T dK~
    store_vec<KC>(static_cast<bf16_t*>(PART == 1 ? a.dv : a.dk) + kv_off, acc);
    if constexpr (BOTH) store_vec<KC>(static_cast<bf16_t*>(a.dv) + kv_off, accv);
  }
}

// Order of the key-pass tiles: a launch of `halves` kinds of workgroup (dK
// and dV, or one kind doing both) over T = nseq * nblk * nch tiles each.
// Every XCD takes the same share of each kind, its dK tiles first and then
// the dV tiles of the same sequences, so dV workgroups start on the CUs
// that dK workgroups leave (page-1 key pass 146 -> 137 us, Christoffel
// 298 -> 266 us against two launches) and no XCD holds only the cheaper
// kind (with the kinds split across the XCDs, 89.7 -> 86.4 us).  Within a
// kind an XCD runs its tiles block rank by block rank across its sequences,
// longest first: key block 0 is reached by every offset, later blocks by
// fewer (86.4 -> 82.6 us).  Without whole sequences per XCD, each kind
// runs sequence by sequence.
struct KeyTile {
  int part, tile;
};
__device__ __forceinline__ KeyTile key_tile_order(int bid, int T, int halves, int nblk, int nch) {
  const int total = halves * T;
  const int t = xcd_tile(bid, total);
  if (T % kNumXcd != 0) return {t >= T ? 1 : 0, t >= T ? t - T : t};
  const int h = T / kNumXcd, per = halves * h;
  const int x = t / per, r = t - x * per;
  const int part = r >= h ? 1 : 0, rr = r - part * h;
  const int spx = h / (nblk * nch);  // sequences per XCD
  int tile = x * h + rr;
  if (spx * nblk * nch == h) {
    const int rank = rr / (spx * nch), rem = rr - rank * (spx * nch);
    tile = ((x * spx + rem / nch) * nblk + rank) * nch + rem % nch;
  }
  return {part, tile};
}

// With the offset gradient requested the launch leads with kNumXcd more
// workgroups: the first reduces dd and dtheta (the query pass, which wrote
// their partials, has finished), concurrently with the key tiles instead of
// as a kernel after them; the others return at once, so every key tile
// keeps its XCD.
template <int D, int G>
__global__ __launch_bounds__(kKeyBlockH16) void bwd_key_h16_kernel(BwdArgs a, StepTable st, ReduceArgs ra) {
  int bid = blockIdx.x;
  if (ra.n_rungs > 0) {
    if (bid < kNumXcd) {
      extern __shared__ __align__(16) uint32_t key_smem[];
      if (bid == 0) reduce_body(ra, reinterpret_cast<double*>(key_smem), kKeyBlockH16);
      return;
    }
    bid -= kNumXcd;
  }
  constexpr int NCH = D / key_chunk_h16(D, G);
  if constexpr (G == 1) {
    key_half_body<D, 1, 2>(a, st, key_tile_order(bid, a.tiles, 1, a.nblk, NCH).tile);  // both halves
  } else {
    const KeyTile kt = key_tile_order(bid, a.tiles, 2, a.nblk, NCH);
    if (kt.part == 0)
      key_half_body<D, G, 0>(a, st, kt.tile);
    else
      key_half_body<D, G, 1>(a, st, kt.tile);
  }
}

// Lanes per query in bwd_query.  The LDS of a workgroup is fixed by its
// stage rows, so more lanes per query put more waves on a CU; that pays
// where the G x DC register tiles are large: with G >= 4 a lane takes 4 dims
// (D = 64, G = 4: 16 lanes, 117 VGPRs, 4 waves per SIMD, against 8 lanes,
// 192 VGPRs and 2 waves), with fewer heads 8 dims (there a lane's dot is so
// short that the extra reduction steps cost more than the waves gain).  At
// least two lanes per head, never fewer than 2 dims (rotation pairs) or more
// than 16 lanes.
template <int D, int G>
constexpr int bwd_lpq() {
  constexpr int dims = G >= 4 ? 4 : 8;
  constexpr int a = 2 * G > D / dims ? 2 * G : D / dims;
  constexpr int b = a < D / 2 ? a : D / 2;
  return b < 16 ? b : 16;
}

// Lanes per query in bwd_edges_query (keys straight from global memory):
// at most 8 dims per lane, same other limits.
template <int D, int G>
constexpr int edge_lpq() {
  constexpr int a = 2 * G > D / 8 ? 2 * G : D / 8;
  constexpr int b = a < D / 2 ? a : D / 2;
  return b < 16 ? b : 16;
}

BwdArgs make_args(const Problem& p, const SlotTable& t, const BwdWorkspace& ws) {
  BwdArgs a{};
  a.P = ws.p;
  a.dP = ws.dp;
  a.Dvec = ws.dvec;
  a.Linv = ws.linv;
  a.dd_part = ws.dd_part;
  a.xq = ws.xq;
  a.xd = ws.xd;
  a.wmax = ws.wmax;
  a.rope = p.rope;
  a.n = p.n;
  a.hq = p.hq;
  a.hkv = p.hkv;
  a.nblk = 1;  // each launcher sets its own blocks per sequence; tiles / nblk = sequences
  a.tiles = p.B * p.hkv;
  a.S = t.count;
  a.n_rungs = t.n_rungs;
  a.scale = p.scale;
  a.scale_log2 = p.scale * kLog2e;
  return a;
}

// dd registers per lane of bwd_query: the small variant holds 16 rungs
// (the Fibonacci and power-of-2 bases), the large one 16 x ND (ND = LPQ / G
// duplicate lanes per query head); more rungs take one launch per window of
// 16 x ND (every launch writes the same dQ and workspace, and the dd
// partials of its own rungs).
template <int D, int G>
constexpr int bwd_rpl_small() {
  constexpr int nd = bwd_lpq<D, G>() / G;
  return nd >= 16 ? 1 : 16 / nd;
}
constexpr int kRplLarge = 16;

template <typename T, int D, int G>
int launch_query_t(const BwdArgs& a0, const SlotTable& t, hipStream_t st) {
  constexpr int LPQ = bwd_lpq<D, G>();
  constexpr int BQ = bwd_bq<G>();
  constexpr int ND = LPQ / G;
  constexpr int RS = bwd_rpl_small<D, G>();
  BwdArgs a = a0;
  a.nblk = (a.n + BQ - 1) / BQ;
  a.tiles = a.nblk * (a0.tiles / a0.nblk);
  const bool dd = a.want_dd && t.n_rungs > 0;
  a.want_dd = dd ? 1 : 0;
  a.r0 = 0;
  // Without the offset gradient the RPL = 0 instantiation runs, in which
  // the rung checks, the dd rows' bookkeeping and the dd registers fold away
  // at compile time (Christoffel query pass 148.3 -> 127.9 us causal,
  // 312 -> 268 us bidirectional, against the dd-capable kernel with the
  // gradient switched off at run time).
  if (!dd) {
    SFA_LAUNCH((bwd_query_kernel<T, D, G, LPQ, bwd_query_cap<T, G, 0>(), BQ, 0>), dim3(a.tiles), dim3(BQ * LPQ), 0, st, a, t);
    return int(hipGetLastError());
  }
  if (t.n_rungs <= RS * ND) {
    SFA_LAUNCH((bwd_query_kernel<T, D, G, LPQ, bwd_query_cap<T, G, RS>(), BQ, RS>), dim3(a.tiles), dim3(BQ * LPQ), 0, st, a, t);
    return int(hipGetLastError());
  }
  for (int r0 = 0; r0 < t.n_rungs; r0 += kRplLarge * ND) {
    a.r0 = r0;
    SFA_LAUNCH((bwd_query_kernel<T, D, G, LPQ, bwd_query_cap<T, G, kRplLarge>(), BQ, kRplLarge>), dim3(a.tiles), dim3(BQ * LPQ), 0, st,
                       a, t);
    if (hipError_t e = hipGetLastError()) return int(e);
  }
  return 0;
}

template <typename T, int D, int G>
int launch_key_t(const BwdArgs& a0, const SlotTable& t, const ReduceArgs* ra, hipStream_t st) {
  BwdArgs a = a0;
  if constexpr (sizeof(T) == 2) {
    constexpr int KB = kKeyBlockH16;
    a.nblk = (a.n + KB - 1) / KB;
    a.tiles = a.nblk * (a0.tiles / a0.nblk) * (D / key_chunk_h16(D, G));
    a.kcap = key_half_cap(G, D);
    const size_t lds = size_t(a.kcap) * key_half_row_words(G, D) * 4;
    const StepTable steps = make_step_table(t, a.n);
    static_assert(sizeof(double) * SFA_MAX_OFFSETS <= size_t(kKeyBlockH16 + 12) * 4 * key_half_row_words(G, D),
                  "the reduce workgroup's doubles fit the key pass's LDS");
    ReduceArgs r{};  // n_rungs = 0: no reduce workgroups
    if (ra) r = *ra;
    const int grid = (G == 1 ? a.tiles : 2 * a.tiles) + (r.n_rungs > 0 ? kNumXcd : 0);
    SFA_LAUNCH((bwd_key_h16_kernel<D, G>), dim3(grid), dim3(KB), lds, st, a, steps, r);
  } else {
    constexpr int KB = key_block(sizeof(T), G, D);
    a.nblk = (a.n + KB - 1) / KB;
    a.tiles = a.nblk * (a0.tiles / a0.nblk) * (D / key_chunk(D));
    SFA_LAUNCH((bwd_key_kernel<T, D, G>), dim3(a.tiles), dim3(KB), 0, st, a, t);
  }
  return int(hipGetLastError());
}

#define SFA_DISPATCH_G(T, D_, FN, g_, ...)         \
  do {                                             \
    if (g_ == 1) return FN<T, D_, 1>(__VA_ARGS__); \
    if (g_ == 2) return FN<T, D_, 2>(__VA_ARGS__); \
    if (g_ == 4) return FN<T, D_, 4>(__VA_ARGS__); \
    return FN<T, D_, 8>(__VA_ARGS__);              \
  } while (0)
#define SFA_DISPATCH_D(T, FN, d_, g_, ...)                       \
  do {                                                           \
    if (d_ == 64) SFA_DISPATCH_G(T, 64, FN, g_, __VA_ARGS__);    \
    else if (d_ == 32) SFA_DISPATCH_G(T, 32, FN, g_, __VA_ARGS__); \
    else SFA_DISPATCH_G(T, 16, FN, g_, __VA_ARGS__);             \
  } while (0)
// bf16 tensors also come with 128 dims (fp32 ones are refused there).
#define SFA_DISPATCH(FN, P, ...)                                 \
  do {                                                           \
    if ((P).dtype == SFA_BF16 && (P).D == 128) SFA_DISPATCH_G(bf16_t, 128, FN, (P).G, __VA_ARGS__); \
    if ((P).dtype == SFA_BF16) SFA_DISPATCH_D(bf16_t, FN, (P).D, (P).G, __VA_ARGS__); \
    else SFA_DISPATCH_D(float, FN, (P).D, (P).G, __VA_ARGS__);   \
  } while (0)


// ------------------------------------------------------- edge-list backward
// Training with per-query key lists ("Critical power-law sparse attention",
// item 4; "Christoffel-Balanced Sparse Attention"): gradients of
// L = <O, dO> for the edge-list forward, one plain key per slot.
//
// bwd_edges_query: per query, the same lane layout as the offset query pass
//   with keys read straight from global memory (L2-resident per KV head):
//   p = exp(logit - lse), dp = dO . v_j, Dvec = sum p dp, dq~ = scale
//   (sum p dp k~_j - Dvec sum p k~_j); p and dp of every valid slot go to
//   the workspace.
// bwd_edges_key: per key j (one lane, 16 dims), the slots that name j from
//   the inverted table in ascending order: dK~_j = sum R(i) scale sum_h dS_h
//   q_h(i), dV_j = sum sum_h p_h dO_h(i); dK = R(j)^T dK~.  No atomics, fixed
//   order.
struct EdgeBwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* lse;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* P;     // [B*Hkv][n][width][G]
  float* dP;    // [B*Hkv][n][width][G]
  float* Dvec;  // [B*Hkv][n][G] Dvec / l
  float* Linv;  // [B*Hkv][n][G] 1 / l, l = sum over the list of p
  const float* rope;
  const int32_t* edges;
  const int32_t* count;
  const int32_t* inv;
  const int32_t* inv_count;
  int width, inv_width;
  int width_shift;  // log2(width) when width is a power of two, else -1
  int n, hq, hkv, nblk, tiles;
  float scale, scale_log2;
};

constexpr int kEdgeBQ = 32;  // queries per bwd_edges_query workgroup
constexpr int kEdgeKB = 64;  // lanes per bwd_edges_key workgroup (one wave)

template <typename T, int D, int G, int LPQ>
__global__ __launch_bounds__(kEdgeBQ* LPQ) void bwd_edges_query_kernel(EdgeBwdArgs a) {
  constexpr int DC = D / LPQ;
  const int tid = threadIdx.x;
  const int qq = tid / LPQ;
  const int c = tid % LPQ;
  using HS = HeadSlice<G, LPQ>;
  const int own = HS::own(c);
  const int tile = xcd_tile(blockIdx.x, a.tiles);
  const int seq = tile / a.nblk;
  const int blk = tile % a.nblk;
  const int b = seq / a.hkv, g = seq % a.hkv;
  const int n = a.n;
  const int i = blk * kEdgeBQ + qq;
  const bool active = i < n;

  const T* __restrict__ Q = static_cast<const T*>(a.q);
  const T* __restrict__ dO = static_cast<const T*>(a.dout);
  const size_t kv_row = size_t(a.hkv) * D;
  const T* Kseq = static_cast<const T*>(a.k) + size_t(b) * n * kv_row + size_t(g) * D + c * DC;
  const T* Vseq = static_cast<const T*>(a.v) + size_t(b) * n * kv_row + size_t(g) * D + c * DC;

  float qv[G][DC], dov[G][DC], acc_pd[G][DC], acc_p[G][DC];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (active) {
      const size_t off = ((size_t(b) * n + i) * a.hq + size_t(g) * G + HS::head(c, h)) * D + c * DC;
      load_vec<DC>(Q + off, qv[h]);
      if (a.rope) rotate_pairs<DC, 1>(qv[h], a.rope + size_t(i) * D, c * DC);
      load_vec<DC>(dO + off, dov[h]);
    } else {
#pragma unroll
      for (int x = 0; x < DC; ++x) qv[h][x] = dov[h][x] = 0.f;
    }
#pragma unroll
    for (int x = 0; x < DC; ++x) acc_pd[h][x] = acc_p[h][x] = 0.f;
  }
  const float lse2 = active ? a.lse[(size_t(b) * a.hq + size_t(g) * G + own) * n + i] * kLog2e : 0.f;
  const int cnt = active ? min(a.count[i], a.width) : 0;
  int cmax = cnt;  // wave-uniform trip count: the longest list of the wavefront
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) cmax = max(cmax, __shfl_xor(cmax, msk));
  const int32_t* erow = a.edges + size_t(active ? i : 0) * a.width;
  const size_t wrow = (size_t(seq) * n + (active ? i : 0)) * a.width;
  float dvec = 0.f;
  float psum = 0.f;  // l = sum p (1 up to the forward's lse)

  // Branch-free over the wave's longest list: a padding entry (or a key
  // outside [0, n)) reads row 0 and is masked by p = 0.  Entries run in
  // chunks of ECH: the K and V rows of a chunk are requested together as
  // raw words (converted where they are used), so the chunk waits for its
  // gathered rows once, and the list entries of the next chunk are read
  // with them, off the chunk's dependency chain (power-law query side
  // 42.2 -> 39.7 us against one entry of rows loaded ahead).
  auto row_of = [&](int t) {
    const int key = t < cnt ? erow[min(t, a.width - 1)] : -1;
    return (key >= 0 && key < n) ? key : -1;  // -1: masked
  };
  constexpr int EW = DC * int(sizeof(T)) / 4;  // 32-bit words of a lane's row chunk
  constexpr int ECH = 4;
  int keys[ECH];
#pragma unroll
  for (int j = 0; j < ECH; ++j) keys[j] = row_of(j);
  for (int t0 = 0; t0 < cmax; t0 += ECH) {
    uint32_t kw[ECH][EW], vw[ECH][EW];
#pragma unroll
    for (int j = 0; j < ECH; ++j) {
      const size_t r = size_t(max(keys[j], 0)) * kv_row;
      load_words<EW>(reinterpret_cast<const uint32_t*>(Kseq + r), kw[j]);
      load_words<EW>(reinterpret_cast<const uint32_t*>(Vseq + r), vw[j]);
    }
    int knext[ECH];
#pragma unroll
    for (int j = 0; j < ECH; ++j) knext[j] = row_of(t0 + ECH + j);
#pragma unroll
    for (int j = 0; j < ECH; ++j) {
      const int t = t0 + j;
      if (t >= cmax) break;  // uniform
      const bool valid = keys[j] >= 0;
      const int kc = valid ? keys[j] : 0;
      float kt[DC], vt[DC];
      words_to_floats<T, DC>(kw[j], kt);
      words_to_floats<T, DC>(vw[j], vt);
      if (a.rope) rotate_pairs<DC, 1>(kt, a.rope + size_t(kc) * D, c * DC);
      const float sdot = own_dot<G, LPQ, DC>(qv, kt);
      const float dp = own_dot<G, LPQ, DC>(dov, vt);
      const float ex = __builtin_amdgcn_exp2f(sdot * a.scale_log2 - lse2);
      const float p = valid ? ex : 0.f;
      const float pdp = p * dp;
      dvec += pdp;
      psum += p;
      if (valid && HS::writer(c)) {
        a.P[(wrow + t) * G + own] = p;
        a.dP[(wrow + t) * G + own] = dp;
      }
      float ph[G], pdh[G];
      HS::bcast(p, ph);
      HS::bcast(pdp, pdh);
#pragma unroll
      for (int h = 0; h < G; ++h)
#pragma unroll
        for (int x = 0; x < DC; ++x) {
          acc_pd[h][x] = fmaf(pdh[h], kt[x], acc_pd[h][x]);
          acc_p[h][x] = fmaf(ph[h], kt[x], acc_p[h][x]);
        }
    }
#pragma unroll
    for (int j = 0; j < ECH; ++j) keys[j] = knext[j];
  }

  // p relative to l = sum p, as in the offset query pass
  const float linv = psum > 0.f ? 1.f / psum : 0.f;
  const float dvn = dvec * linv;
  if (active && HS::writer(c)) {
    a.Dvec[(size_t(seq) * n + i) * G + own] = dvn;
    a.Linv[(size_t(seq) * n + i) * G + own] = linv;
  }
  float dvh[G], slh[G];
  HS::bcast(dvn, dvh);
  HS::bcast(a.scale * linv, slh);
  if (active) {
    T* dQ = static_cast<T*>(a.dq);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float dq[DC];
#pragma unroll
      for (int x = 0; x < DC; ++x) dq[x] = slh[h] * fmaf(-dvh[h], acc_p[h][x], acc_pd[h][x]);
      if (a.rope) rotate_pairs<DC, -1>(dq, a.rope + size_t(i) * D, c * DC);
      store_vec<DC>(dQ + ((size_t(b) * n + i) * a.hq + size_t(g) * G + HS::head(c, h)) * D + c * DC, dq);
    }
  }
}

// One wave holds all D / KC chunks of kEdgeKB / (D / KC) keys (lane = key x
// chunk), so the chunk lanes of a key read one whole head row of Q and dO
// together and share its list entry and P, dP, Dvec loads.
template <typename T, int D, int G>
__global__ __launch_bounds__(kEdgeKB) void bwd_edges_key_kernel(EdgeBwdArgs a) {
  constexpr int KC = key_chunk(D);
  constexpr int NCH = D / KC;
  constexpr int KPW = kEdgeKB / NCH;  // keys per workgroup
  const int tid = threadIdx.x;
  const int tile = xcd_tile(blockIdx.x, a.tiles);
  const int c = tid % NCH;
  const int seq = tile / a.nblk;
  const int blk = tile % a.nblk;
  const int b = seq / a.hkv, g = seq % a.hkv;
  const int n = a.n;
  const int j = blk * KPW + tid / NCH;
  const bool activej = j < n;

  const T* __restrict__ Q = static_cast<const T*>(a.q);
  const T* __restrict__ dO = static_cast<const T*>(a.dout);
  const int cnt = activej ? min(a.inv_count[j], a.inv_width) : 0;
  int cmax = cnt;
#pragma unroll
  for (int msk = 1; msk < 64; msk <<= 1) cmax = max(cmax, __shfl_xor(cmax, msk));
  const int32_t* irow = a.inv + size_t(activej ? j : 0) * a.inv_width;
  const int64_t nslots = int64_t(n) * a.width;

  float ak[KC], av[KC];
#pragma unroll
  for (int x = 0; x < KC; ++x) ak[x] = av[x] = 0.f;
  // Branch-free over the wave's longest list: an entry past the lane's
  // count, or one that is not a slot of the table, reads slot 0 and enters
  // with zero weights.  Entries run in chunks of ECH: the loads of a chunk
  // (each entry's P, dP, Dvec, 1/l and, with one head per KV head, its Q and
  // dO rows as raw words) are issued together, so the chunk waits for its
  // gathered data once, and the list entries of the next chunk are read
  // with them.  (With more heads the rows of a chunk would not fit the
  // registers; there the rows are loaded in the step.)  A slot s of the
  // table is query s / width, entry s % width: a shift when the width is a
  // power of two, as in the power-law layer.  (Power-law key side 42.2 ->
  // 38.3 us against one entry loaded ahead; chunks of 4 took 39.3 us, their
  // registers costing a wave per SIMD.)
  constexpr bool kRowsAhead = G == 1;
  constexpr int ECH = 2;
  constexpr int QW = KC * int(sizeof(T)) / 4;  // 32-bit words of a lane's row chunk
  auto entry_at = [&](int u) { return u < cnt ? irow[min(u, a.inv_width - 1)] : -1; };
  int ents[ECH];
#pragma unroll
  for (int k = 0; k < ECH; ++k) ents[k] = entry_at(k);
  for (int u0 = 0; u0 < cmax; u0 += ECH) {
    int iq[ECH];
    bool okq[ECH];
    float pg[ECH][G], dpg[ECH][G], dvg[ECH][G], lg[ECH][G];
    uint32_t qw[kRowsAhead ? ECH : 1][QW], ow[kRowsAhead ? ECH : 1][QW];
#pragma unroll
    for (int k = 0; k < ECH; ++k) {
      const int e = ents[k];
      okq[k] = e >= 0 && e < nslots;
      const int ec = okq[k] ? e : 0;
      const int i = a.width_shift >= 0 ? (ec >> a.width_shift) : ec / a.width;
      iq[k] = i;
      const int t = ec - i * a.width;
      const size_t w = ((size_t(seq) * n + i) * a.width + t) * G;
      load_vec<G>(a.P + w, pg[k]);
      load_vec<G>(a.dP + w, dpg[k]);
      load_vec<G>(a.Dvec + (size_t(seq) * n + i) * G, dvg[k]);
      load_vec<G>(a.Linv + (size_t(seq) * n + i) * G, lg[k]);
      if constexpr (kRowsAhead) {
        const size_t off = ((size_t(b) * n + i) * a.hq + size_t(g) * G) * D + c * KC;
        load_words<QW>(reinterpret_cast<const uint32_t*>(Q + off), qw[k]);
        load_words<QW>(reinterpret_cast<const uint32_t*>(dO + off), ow[k]);
      }
    }
    int enext[ECH];
#pragma unroll
    for (int k = 0; k < ECH; ++k) enext[k] = entry_at(u0 + ECH + k);
#pragma unroll
    for (int k = 0; k < ECH; ++k) {
      if (u0 + k >= cmax) break;  // uniform
      const int i = iq[k];
      float yk[KC], yv[KC];
#pragma unroll
      for (int x = 0; x < KC; ++x) yk[x] = yv[x] = 0.f;
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float pgl = pg[k][h] * lg[k][h];  // p / l
        const float ds = okq[k] ? a.scale * pgl * (dpg[k][h] - dvg[k][h]) : 0.f;
        const float pw = okq[k] ? pgl : 0.f;
        float qx[KC], ox[KC];
        if constexpr (kRowsAhead) {
          words_to_floats<T, KC>(qw[k], qx);
          words_to_floats<T, KC>(ow[k], ox);
        } else {
          const size_t off = ((size_t(b) * n + i) * a.hq + size_t(g) * G + h) * D + c * KC;
          load_vec<KC>(Q + off, qx);
          load_vec<KC>(dO + off, ox);
        }
#pragma unroll
        for (int x = 0; x < KC; ++x) {
          yk[x] = fmaf(ds, qx[x], yk[x]);
          yv[x] = fmaf(pw, ox[x], yv[x]);
        }
      }
      if (a.rope) rotate_pairs<KC, 1>(yk, a.rope + size_t(i) * D, c * KC);  // into the frame of position i
#pragma unroll
      for (int x = 0; x < KC; ++x) {
        ak[x] += yk[x];
        av[x] += yv[x];
      }
    }
#pragma unroll
    for (int k = 0; k < ECH; ++k) ents[k] = enext[k];
  }
  if (activej) {
    if (a.rope) rotate_pairs<KC, -1>(ak, a.rope + size_t(j) * D, c * KC);  // dK = R(j)^T dK~
    const size_t kv_off = (size_t(b) * n + j) * size_t(a.hkv) * D + size_t(g) * D + c * KC;
    store_vec<KC>(static_cast<T*>(a.dk) + kv_off, ak);
    store_vec<KC>(static_cast<T*>(a.dv) + kv_off, av);
  }
}

template <typename T, int D, int G>
int launch_edges_t(const EdgeBwdArgs& a0, hipStream_t st) {
  constexpr int LPQ = edge_lpq<D, G>();
  EdgeBwdArgs a = a0;
  const int seqs = a0.tiles;  // B * hkv on entry
  {
    ProfileScope ps("bwd_edges_query", st);
    a.nblk = (a.n + kEdgeBQ - 1) / kEdgeBQ;
    a.tiles = a.nblk * seqs;
    SFA_LAUNCH((bwd_edges_query_kernel<T, D, G, LPQ>), dim3(a.tiles), dim3(kEdgeBQ * LPQ), 0, st, a);
  }
  if (hipError_t e = hipGetLastError()) return int(e);
  {
    ProfileScope ps("bwd_edges_key", st);
    constexpr int KPW = kEdgeKB / (D / key_chunk(D));
    a.nblk = (a.n + KPW - 1) / KPW;
    a.tiles = a.nblk * seqs;
    SFA_LAUNCH((bwd_edges_key_kernel<T, D, G>), dim3(a.tiles), dim3(kEdgeKB), 0, st, a);
  }
  return int(hipGetLastError());
}

}  // namespace

size_t bwd_workspace_layout(const Problem& p, const SlotTable& t, void* base, BwdWorkspace* ws) {
  auto al = [](size_t e) { return (e + 63) & ~size_t(63); };  // 256-byte aligned sections
  const size_t pe = al(size_t(p.B) * p.hkv * t.count * size_t(p.n) * p.G);  // floats per array
  const size_t de = al(size_t(p.B) * p.hkv * size_t(p.n) * p.G);
  // dd partials per rung: one per query-pass workgroup
  const bool h16 = p.dtype == SFA_BF16;
  const int bq = p.G >= 4 ? bwd_bq<4>() : bwd_bq<1>();
  ws->blocks = ((p.n + bq - 1) / bq) * p.B * p.hkv;
  const size_t dd_e = al(size_t(ws->blocks) * (t.n_rungs > 0 ? t.n_rungs : 1));
  // packed key-pass rows (bf16, G >= 2): D * G / 2 words per (sequence, row)
  const size_t xe = (h16 && p.G >= 2) ? al(size_t(p.B) * p.hkv * size_t(p.n) * p.D * (p.G / 2)) : 0;
  // dS bounds (bf16, G >= 2): one per query-pass workgroup
  const size_t we = (h16 && p.G >= 2) ? al(size_t(ws->blocks)) : 0;
  float* f = static_cast<float*>(base);
  ws->p = f;
  ws->dp = f ? f + pe : nullptr;
  ws->dvec = f ? f + 2 * pe : nullptr;
  ws->linv = f ? f + 2 * pe + de : nullptr;
  ws->dd_part = f ? f + 2 * pe + 2 * de : nullptr;
  ws->xq = (f && xe) ? reinterpret_cast<uint32_t*>(f + 2 * pe + 2 * de + dd_e) : nullptr;
  ws->xd = (f && xe) ? reinterpret_cast<uint32_t*>(f + 2 * pe + 2 * de + dd_e + xe) : nullptr;
  ws->wmax = (f && we) ? f + 2 * pe + 2 * de + dd_e + 2 * xe : nullptr;
  ws->bytes = (2 * pe + 2 * de + dd_e + 2 * xe + we) * sizeof(float);
  return ws->bytes;
}

int launch_bwd_query(const Problem& p, const SlotTable& t, const void* q, const void* k, const void* v,
                     const float* lse, const void* dout, void* dq, const BwdWorkspace& ws, bool want_dd,
                     void* stream) {
  BwdArgs a = make_args(p, t, ws);
  a.want_dd = want_dd ? 1 : 0;
  a.q = q;
  a.k = k;
  a.v = v;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  hipStream_t st = static_cast<hipStream_t>(stream);
  SFA_DISPATCH(launch_query_t, p, a, t, st);
}

void fill_reduce_args(ReduceArgs* a, const SlotTable& t, const BwdWorkspace& ws, const float* base_f, double alpha,
                      float* dd, float* dtheta) {
  a->dd_part = ws.dd_part;
  a->dd = dd;
  a->dtheta = dtheta;
  a->blocks = ws.blocks;
  a->n_rungs = t.n_rungs;
  a->alpha = alpha;
  for (int k = 0; k < t.n_rungs; ++k) a->base[k] = base_f[k];
}

int launch_bwd_key(const Problem& p, const SlotTable& t, const void* q, const void* k, const void* v,
                   const void* dout, void* dk, void* dv, const BwdWorkspace& ws, const float* base_f,
                   double alpha, float* dd, float* dtheta, void* stream) {
  BwdArgs a = make_args(p, t, ws);
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = dout;
  a.dk = dk;
  a.dv = dv;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // bf16: dd and dtheta are reduced by a leading workgroup of the key pass
  ReduceArgs r{};
  const bool fold = p.dtype == SFA_BF16 && (dd || dtheta) && t.n_rungs > 0;
  if (fold) fill_reduce_args(&r, t, ws, base_f, alpha, dd, dtheta);
  SFA_DISPATCH(launch_key_t, p, a, t, fold ? &r : nullptr, st);
}

bool bwd_key_reduces(const Problem& p, const SlotTable& t, bool want) {
  return p.dtype == SFA_BF16 && want && t.n_rungs > 0;
}

int launch_bwd_reduce(const SlotTable& t, const BwdWorkspace& ws, const float* base_f, double alpha, float* dd,
                      float* dtheta, void* stream) {
  ReduceArgs a{};
  fill_reduce_args(&a, t, ws, base_f, alpha, dd, dtheta);
  SFA_LAUNCH(bwd_reduce_kernel, dim3(1), dim3(kReduceThreads), 0, static_cast<hipStream_t>(stream), a);
  return int(hipGetLastError());
}

size_t bwd_edges_workspace_layout(const Problem& p, int width, void* base, float** P, float** dP, float** Dvec,
                                  float** Linv) {
  auto al = [](size_t e) { return (e + 63) & ~size_t(63); };
  const size_t pe = al(size_t(p.B) * p.hkv * size_t(p.n) * size_t(width) * p.G);
  const size_t de = al(size_t(p.B) * p.hkv * size_t(p.n) * p.G);
  float* f = static_cast<float*>(base);
  if (P) *P = f;
  if (dP) *dP = f ? f + pe : nullptr;
  if (Dvec) *Dvec = f ? f + 2 * pe : nullptr;
  if (Linv) *Linv = f ? f + 2 * pe + de : nullptr;
  return (2 * pe + 2 * de) * sizeof(float);
}

int launch_bwd_edges(const Problem& p, const int32_t* edges, const int32_t* count, int width, const int32_t* inv,
                     const int32_t* inv_count, int inv_width, const void* q, const void* k, const void* v,
                     const float* lse, const void* dout, void* dq, void* dk, void* dv, void* workspace,
                     void* stream) {
  EdgeBwdArgs a{};
  a.q = q;
  a.k = k;
  a.v = v;
  a.lse = lse;
  a.dout = dout;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  bwd_edges_workspace_layout(p, width, workspace, &a.P, &a.dP, &a.Dvec, &a.Linv);
  a.rope = p.rope;
  a.edges = edges;
  a.count = count;
  a.inv = inv;
  a.inv_count = inv_count;
  a.width = width;
  a.inv_width = inv_width;
  a.width_shift = -1;
  for (int sh = 0; sh < 31; ++sh)
    if ((1 << sh) == width) a.width_shift = sh;
  a.n = p.n;
  a.hq = p.hq;
  a.hkv = p.hkv;
  a.nblk = 1;
  a.tiles = p.B * p.hkv;
  a.scale = p.scale;
  a.scale_log2 = p.scale * kLog2e;
  hipStream_t st = static_cast<hipStream_t>(stream);
  SFA_DISPATCH(launch_edges_t, p, a, st);
}

}  // namespace sfa
