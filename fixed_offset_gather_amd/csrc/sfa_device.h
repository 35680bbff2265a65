// Device-side helpers for the gfx950 kernels of libsfa: bf16 conversion,
// vector loads/stores into float registers, cross-lane group reductions on
// 64-wide wavefronts (DPP where the group fits in a 16-lane row), rotary
// rotation of interleaved pairs and the XCD-aware tile order.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace sfa {

typedef uint16_t bf16_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNumXcd = 8;

__device__ __forceinline__ float neg_inf() { return -__builtin_huge_valf(); }

// bfloat16 is the upper half of an IEEE float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bfloat16 bits (low half = lo), round to nearest
// even: one v_cvt_pk_bf16_f32.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- loads

// N consecutive elements of T at p (N * sizeof(T) bytes, naturally aligned
// to the widest vector used) widened to float.
template <int N>
__device__ __forceinline__ void load_vec(const float* __restrict__ p, float (&out)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int x = 0; x < N; x += 4) {
      const float4 t = *reinterpret_cast<const float4*>(p + x);
      out[x] = t.x; out[x + 1] = t.y; out[x + 2] = t.z; out[x + 3] = t.w;
    }
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int x = 0; x < N; x += 2) {
      const float2 t = *reinterpret_cast<const float2*>(p + x);
      out[x] = t.x; out[x + 1] = t.y;
    }
  } else {
#pragma unroll
    for (int x = 0; x < N; ++x) out[x] = p[x];
  }
}

template <int N>
__device__ __forceinline__ void load_vec(const bf16_t* __restrict__ p, float (&out)[N]) {
  if constexpr (N % 8 == 0) {
#pragma unroll
    for (int x = 0; x < N; x += 8) {
      const uint4 t = *reinterpret_cast<const uint4*>(p + x);
      out[x] = bf16_lo(t.x); out[x + 1] = bf16_hi(t.x);
      out[x + 2] = bf16_lo(t.y); out[x + 3] = bf16_hi(t.y);
      out[x + 4] = bf16_lo(t.z); out[x + 5] = bf16_hi(t.z);
      out[x + 6] = bf16_lo(t.w); out[x + 7] = bf16_hi(t.w);
    }
  } else if constexpr (N % 4 == 0) {
#pragma unroll
    for (int x = 0; x < N; x += 4) {
      const uint2 t = *reinterpret_cast<const uint2*>(p + x);
      out[x] = bf16_lo(t.x); out[x + 1] = bf16_hi(t.x);
      out[x + 2] = bf16_lo(t.y); out[x + 3] = bf16_hi(t.y);
    }
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int x = 0; x < N; x += 2) {
      const uint32_t t = *reinterpret_cast<const uint32_t*>(p + x);
      out[x] = bf16_lo(t); out[x + 1] = bf16_hi(t);
    }
  } else {
#pragma unroll
    for (int x = 0; x < N; ++x) out[x] = __uint_as_float(uint32_t(p[x]) << 16);
  }
}

// N elements of T held as raw 32-bit words (N * sizeof(T) / 4 of them),
// widened to float.
template <typename T, int N>
__device__ __forceinline__ void words_to_floats(const uint32_t (&w)[N * sizeof(T) / 4], float (&out)[N]) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int x = 0; x < N / 2; ++x) {
      out[2 * x] = bf16_lo(w[x]);
      out[2 * x + 1] = bf16_hi(w[x]);
    }
  } else {
#pragma unroll
    for (int x = 0; x < N; ++x) out[x] = __uint_as_float(w[x]);
  }
}

// One element widened to float.
__device__ __forceinline__ float load1(const float* p) { return *p; }
__device__ __forceinline__ float load1(const bf16_t* p) { return __uint_as_float(uint32_t(*p) << 16); }

// N consecutive floats at a uniform base plus a 32-bit per-lane byte offset,
// loaded through the global address space (global_load with an SGPR base).
// The caller keeps `base` uniform; the empty asm keeps the offset a 32-bit
// VGPR at the load (see store_global_at).
template <int N>
__device__ __forceinline__ void load_global_at(const float* base, unsigned byte_off, float (&out)[N]) {
  typedef float v4f __attribute__((ext_vector_type(4)));
  typedef float v2f __attribute__((ext_vector_type(2)));
  typedef __attribute__((address_space(1))) const char gcchar;
  typedef __attribute__((address_space(1))) const v4f gcv4f;
  typedef __attribute__((address_space(1))) const v2f gcv2f;
  typedef __attribute__((address_space(1))) const float gcfloat;
  asm volatile("" : "+v"(byte_off));
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int x = 0; x < N; x += 4) {
      const v4f t = *(gcv4f*)((gcchar*)base + byte_off + 16u * (x / 4));
      out[x] = t.x; out[x + 1] = t.y; out[x + 2] = t.z; out[x + 3] = t.w;
    }
  } else if constexpr (N == 2) {
    const v2f t = *(gcv2f*)((gcchar*)base + byte_off);
    out[0] = t.x; out[1] = t.y;
  } else {
    static_assert(N == 1, "1, 2 or a multiple of 4 floats");
    out[0] = *(gcfloat*)((gcchar*)base + byte_off);
  }
}

// A pointer that is the same in every lane, held in SGPRs (both halves read
// from the first lane), so it can serve as the scalar base of a global
// load or store.
template <typename P>
__device__ __forceinline__ P* uniform_ptr(P* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  return reinterpret_cast<P*>((uint64_t(hi) << 32) | lo);
}

// One float at a uniform base plus a 32-bit per-lane byte offset, stored
// through the global address space (global_store with an SGPR base).
__device__ __forceinline__ void store_global_at(float* base, unsigned byte_off, float v) {
  typedef __attribute__((address_space(1))) char gchar;
  typedef __attribute__((address_space(1))) float gfloat;
  // The empty asm keeps the offset a 32-bit VGPR at the store, so its
  // zero-extension is matched into the instruction instead of being hoisted
  // into a 64-bit register pair.
  asm volatile("" : "+v"(byte_off));
  *(gfloat*)((gchar*)base + byte_off) = v;  // C cast: address-space conversion
}

template <int N>
__device__ __forceinline__ void store_vec(float* __restrict__ p, const float (&in)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int x = 0; x < N; x += 4)
      *reinterpret_cast<float4*>(p + x) = make_float4(in[x], in[x + 1], in[x + 2], in[x + 3]);
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int x = 0; x < N; x += 2) *reinterpret_cast<float2*>(p + x) = make_float2(in[x], in[x + 1]);
  } else {
#pragma unroll
    for (int x = 0; x < N; ++x) p[x] = in[x];
  }
}

template <int N>
__device__ __forceinline__ void store_vec(bf16_t* __restrict__ p, const float (&in)[N]) {
  if constexpr (N % 8 == 0) {
#pragma unroll
    for (int x = 0; x < N; x += 8) {
      uint4 t;
      t.x = pack_bf2(in[x], in[x + 1]);
      t.y = pack_bf2(in[x + 2], in[x + 3]);
      t.z = pack_bf2(in[x + 4], in[x + 5]);
      t.w = pack_bf2(in[x + 6], in[x + 7]);
      *reinterpret_cast<uint4*>(p + x) = t;
    }
  } else if constexpr (N % 4 == 0) {
#pragma unroll
    for (int x = 0; x < N; x += 4) {
      uint2 t;
      t.x = pack_bf2(in[x], in[x + 1]);
      t.y = pack_bf2(in[x + 2], in[x + 3]);
      *reinterpret_cast<uint2*>(p + x) = t;
    }
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int x = 0; x < N; x += 2) *reinterpret_cast<uint32_t*>(p + x) = pack_bf2(in[x], in[x + 1]);
  } else {
#pragma unroll
    for (int x = 0; x < N; ++x) p[x] = bf16_t(pack_bf2(in[x], 0.f) & 0xffffu);
  }
}

// ------------------------------------------------------- packed f16

// Two f16 values in one 32-bit register (low half = even element).
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t pack_h2(float lo, float hi) {
  const half2_t h = {(_Float16)lo, (_Float16)hi};  // round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

__device__ __forceinline__ half2_t as_h2(uint32_t w) { return __builtin_bit_cast(half2_t, w); }

// a.lo*b.lo + a.hi*b.hi + c with f16 products accumulated in fp32.
__device__ __forceinline__ float dot2_h(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2(as_h2(a), as_h2(b), c, false);
}

// The same with bfloat16 halves (each product exact in fp32).
__device__ __forceinline__ float dot2_bf(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

// a + w (b - a) on both halves (packed f16 arithmetic).
__device__ __forceinline__ uint32_t lerp_h2(uint32_t a, uint32_t b, half2_t w) {
  const half2_t x = as_h2(a), y = as_h2(b);
  return __builtin_bit_cast(uint32_t, x + w * (y - x));
}

// fp32 c + p * (f16 element): one mixed-precision FMA, no unpacking.
__device__ __forceinline__ float fma_lo(float p, uint32_t w, float c) { return fmaf(p, (float)as_h2(w).x, c); }
__device__ __forceinline__ float fma_hi(float p, uint32_t w, float c) { return fmaf(p, (float)as_h2(w).y, c); }

// N 32-bit words to p (N * 4 bytes, aligned to the widest vector used).
template <int N>
__device__ __forceinline__ void store_words(uint32_t* __restrict__ p, const uint32_t (&w)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int x = 0; x < N; x += 4) *reinterpret_cast<uint4*>(p + x) = make_uint4(w[x], w[x + 1], w[x + 2], w[x + 3]);
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int x = 0; x < N; x += 2) *reinterpret_cast<uint2*>(p + x) = make_uint2(w[x], w[x + 1]);
  } else {
#pragma unroll
    for (int x = 0; x < N; ++x) p[x] = w[x];
  }
}

template <int N>
__device__ __forceinline__ void load_words(const uint32_t* __restrict__ p, uint32_t (&out)[N]) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int x = 0; x < N; x += 4) {
      const uint4 t = *reinterpret_cast<const uint4*>(p + x);
      out[x] = t.x; out[x + 1] = t.y; out[x + 2] = t.z; out[x + 3] = t.w;
    }
  } else if constexpr (N % 2 == 0) {
#pragma unroll
    for (int x = 0; x < N; x += 2) {
      const uint2 t = *reinterpret_cast<const uint2*>(p + x);
      out[x] = t.x; out[x + 1] = t.y;
    }
  } else {
#pragma unroll
    for (int x = 0; x < N; ++x) out[x] = p[x];
  }
}

// ------------------------------------------------------------- rotation

// Rotate the interleaved pairs of x (dims d0 .. d0+N-1 of a head, d0 even)
// by the angles of table row `row` ([pos][D/2][cos, sin]).  sign = +1
// rotates forward (R), -1 applies the transpose (R^T).
template <int N, int SIGN>
__device__ __forceinline__ void rotate_pairs(float (&x)[N], const float* __restrict__ row, int d0) {
  static_assert(N % 2 == 0, "pairs");
  const float* t = row + d0;  // pair p = d0/2 + j sits at floats d0 + 2j
  float cs[N];
  load_vec<N>(t, cs);
#pragma unroll
  for (int j = 0; j < N; j += 2) {
    const float c = cs[j], s = SIGN > 0 ? cs[j + 1] : -cs[j + 1];
    const float a = x[j], b = x[j + 1];
    x[j] = a * c - b * s;
    x[j + 1] = a * s + b * c;
  }
}

// ------------------------------------------------------- lane exchange

// Lane permutation within rows of 16 lanes.  Every control used here reads
// a valid lane of the same row, so no fill value is needed (bound_ctrl set)
// and the move can fold into the consuming add as a DPP operand.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

constexpr int quad_perm(int a, int b, int c, int d) { return a | (b << 2) | (c << 4) | (d << 6); }
constexpr int kDppRowMirror = 0x140;
constexpr int kDppRowHalfMirror = 0x141;

// Sum over aligned groups of L lanes; every lane of the group gets the sum.
template <int L>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (L >= 2) x += dpp<quad_perm(1, 0, 3, 2)>(x);
  if constexpr (L >= 4) x += dpp<quad_perm(2, 3, 0, 1)>(x);
  if constexpr (L >= 8) x += dpp<kDppRowHalfMirror>(x);
  if constexpr (L >= 16) x += dpp<kDppRowMirror>(x);
  if constexpr (L >= 32) x += __shfl_xor(x, 16);
  if constexpr (L >= 64) x += __shfl_xor(x, 32);
  return x;
}

// Value held by the lanes that own head H, where lane c of a query's
// aligned group of L lanes owns head c % G (L a multiple of G, so the owners
// repeat every G lanes and all owners of one head hold the same value).
// L <= 2: the group is part of a quad.  L >= 4 and G <= 4: one DPP move
// inside the lane's quad, which lies in the lane's own group.  G == 8: the
// quad holding head H is the lane's own quad or its mirror in the 8-lane
// half row, both inside the group.
template <int G, int L, int H>
__device__ __forceinline__ float owner_bcast(float x) {
  static_assert(H < G && L % G == 0, "head in group");
  if constexpr (G == 1) {
    return x;
  } else if constexpr (L == 2) {
    return dpp<quad_perm(H, H, 2 + H, 2 + H)>(x);
  } else if constexpr (G <= 4) {
    return dpp<quad_perm(H, H, H, H)>(x);
  } else {
    static_assert(G == 8, "group size");
    const float v = dpp<quad_perm(H & 3, H & 3, H & 3, H & 3)>(x);
    const float w = dpp<kDppRowHalfMirror>(v);
    return ((__lane_id() >> 2) & 1) == (H >> 2) ? v : w;
  }
}

// Butterfly partner inside aligned groups of SPAN lanes (SPAN <= 16): lane c
// reads lane c ^ (SPAN - 1), one DPP move (mirror, half mirror, quad
// reverse, pair swap).
template <int SPAN>
__device__ __forceinline__ float bfly(float x) {
  static_assert(SPAN == 2 || SPAN == 4 || SPAN == 8 || SPAN == 16, "span");
  if constexpr (SPAN == 16) return dpp<kDppRowMirror>(x);
  else if constexpr (SPAN == 8) return dpp<kDppRowHalfMirror>(x);
  else if constexpr (SPAN == 4) return dpp<quad_perm(3, 2, 1, 0)>(x);
  else return dpp<quad_perm(1, 0, 3, 2)>(x);
}

constexpr int ilog2c(int x) { return x <= 1 ? 0 : 1 + ilog2c(x >> 1); }

// Per-head sums over an aligned group of L lanes that all hold partial sums
// of the same G heads (a reduce-scatter).  Lane c keeps its G partials in a
// lane-specific order: register j holds head head(c, j).  Exchange step t
// (t = 0 widest) pairs lane c with lane c ^ ((L >> t) - 1); the first
// log2(G) steps each send half of the remaining registers and keep the other
// half, the rest add the one remaining register.  A full reduction costs
// log2(L) DPP adds instead of G log2(L), and ends with lane c holding the sum
// of head own(c) = c >> log2(L / G), bit-identical in every lane of that
// head (each add has the same two operands).  bcast spreads one value per
// head back into the lane's register order with G - 1 DPP moves.
template <int G, int L>
struct HeadSlice {
  static_assert(G >= 1 && L >= G && L <= 16 && L % G == 0, "head group");
  static constexpr int S = ilog2c(G);
  static constexpr int SH = ilog2c(L / G);
  static constexpr int NSTEP = ilog2c(L);

  __device__ static int own(int c) { return c >> SH; }
  // One lane per head (for stores of per-head values).
  __device__ static bool writer(int c) { return (c & ((1 << SH) - 1)) == 0; }
  __device__ static int head(int c, int j) {
    int m = 0;
    for (int t = 0; t < S; ++t)
      if ((j >> (S - 1 - t)) & 1) m ^= (L >> t) - 1;
    return (c ^ m) >> SH;
  }

  template <int T = 0>
  __device__ static float reduce(float (&x)[G]) {
    if constexpr (T < S) {
      constexpr int half = G >> (T + 1);
#pragma unroll
      for (int j = 0; j < half; ++j) x[j] += bfly<(L >> T)>(x[j + half]);
      return reduce<T + 1>(x);
    } else if constexpr (T < NSTEP) {
      x[0] += bfly<(L >> T)>(x[0]);
      return reduce<T + 1>(x);
    } else {
      return x[0];
    }
  }

  template <int B = 0>
  __device__ static void fill(float (&out)[G]) {
    if constexpr (B < S) {
#pragma unroll
      for (int j = 1 << B; j < (2 << B); ++j) out[j] = bfly<(L >> (S - 1 - B))>(out[j - (1 << B)]);
      fill<B + 1>(out);
    }
  }
  __device__ static void bcast(float v, float (&out)[G]) {
    out[0] = v;
    fill(out);
  }
};

// Sum over the whole 64-lane wavefront (result valid in every lane).
__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// ------------------------------------------------------- online softmax

// The forward kernels' online softmax keeps a running reference per (query,
// head) and raises it only when some lane of the wave sees a logit more than
// this many log2 units above its reference (one ballot per chunk of slots).
// Below that the weights exp2(s - ref) stay at most 2^8 in fp32, and the
// rescale of the output accumulators (an exp, its spread to the lane's heads
// and a multiply per accumulator) is skipped.  The output is the same up to
// rounding: o and l share the reference, and lse = ref + log2 l.  (Page-1
// learned forward 68.3 -> 65.8 us, Christoffel forward 89.7 -> 85.3 us.)
constexpr float kRescaleSlack = 8.f;

// ------------------------------------------------------------ tile order

// Workgroups are dispatched round-robin over the XCDs.  Give each XCD a
// contiguous range of tiles so that the query blocks of one sequence (which
// read the same K/V rows) share one L2.
__device__ __forceinline__ int xcd_tile(int id, int total) {
  if (total % kNumXcd) return id;
  const int per = total / kNumXcd;
  return (id % kNumXcd) * per + id / kNumXcd;
}

// Sequence and query block of workgroup `id` of a launch of `total` =
// nseq * nblk tiles, longest blocks first.  A block's work grows with its
// position (later queries reach more offsets).  When xcd_tile gives each XCD
// whole sequences, the XCD runs its tiles block rank by block rank across
// those sequences, so all of its longest blocks start before any shorter one
// and its last workgroups are the shortest (against each sequence in turn,
// longest block first: page-1 forward 74.8 -> 70.8 us, its backward query
// pass 155.8 -> 152.2 us, the Christoffel query pass 187 -> 157 us).
// Otherwise each sequence runs longest block first.
// canon = seq * nblk + (nblk - 1 - blk) numbers the tiles independently of
// the order, for per-workgroup results.
struct SeqBlock {
  int seq, blk, canon;
};
__device__ __forceinline__ SeqBlock lpt_seq_block(int id, int total, int nblk) {
  const int tile = xcd_tile(id, total);
  int seq, rank;
  const int per = total / kNumXcd;
  if (total % kNumXcd == 0 && per % nblk == 0) {
    const int k = per / nblk;  // sequences per XCD
    const int r = tile - (tile / per) * per;
    seq = (tile / per) * k + r % k;
    rank = r / k;
  } else {
    seq = tile / nblk;
    rank = tile % nblk;
  }
  return {seq, nblk - 1 - rank, seq * nblk + rank};
}

}  // namespace sfa
