// Internal declarations shared by the host translation units of libsfa.
#pragma once

#include <cstdint>
#include <string>

#include "sfa.h"

namespace sfa {

// Thread-local error message; returns `code` so callers can `return fail(...)`.
int fail(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error();

// Slot table handed to the shared-offset kernels by value.  Slots are the
// window distances 0..W and the offsets, sorted by ascending lo (stable, the
// window first on ties); rung is the caller's offset index or -1.  With
// merging (forward only), slots naming the same (lo, frac) become one entry
// of multiplicity mult: its softmax weight is mult * exp(logit), exactly
// the sum of the identical slots.  One 16-byte record per slot, so a kernel
// reads a slot with one scalar load.
struct Slot {
  int32_t lo;
  float frac;  // +0 for an integer slot (kernels test the bit pattern)
  float mult;
  int32_t rung;
};
struct SlotTable {
  int32_t count;
  int32_t n_rungs;
  int32_t pad_[2];
  Slot s[SFA_MAX_SLOTS];
};

// Kernel launch parameters derived from sfa_attn after validation.
struct Problem {
  int B, n, hq, hkv, D, G, dtype, window, n_off, flags;
  float scale;
  const float* rope;
};

int validate_problem(const sfa_attn* a, Problem* p);
int build_slots(const sfa_attn* a, SlotTable* t, bool merge = false);

// Launchers (defined in the .hip translation units).  They return hipError_t
// as int (0 = success) and never validate: callers have done that.
int launch_fwd_offsets(const Problem& p, const SlotTable& t, const void* q,
                       const void* k, const void* v, void* o, float* lse,
                       void* stream);
int launch_fwd_edges(const Problem& p, const int32_t* edges,
                     const int32_t* count, int width, const void* q,
                     const void* k, const void* v, void* o, float* lse,
                     void* stream);

struct BwdWorkspace {
  float* p;        // [B][Hkv][S][n][G] softmax probabilities (0 where a slot has no row)
  float* dp;       // [B][Hkv][S][n][G] dO . v~
  float* dvec;     // [B][Hkv][n][G] rowsum(dO * O) of p / l: (sum_slots p dp) / l
  float* linv;     // [B][Hkv][n][G] 1 / l, l = sum_slots p (1 up to the forward's lse)
  float* dd_part;  // [n_rungs][blocks] per-block partial sums of dL/dd_k (one per query-pass workgroup)
  // bf16 with G >= 2: the query pass's rows for the key pass, as f16 head
  // pairs in the key pass's LDS row layout, [B][Hkv][n][D/16][G/2][16] words
  // (word = heads (2hp, 2hp+1) of one dim): q rotated by its own position,
  // and dO.  Null otherwise (the key pass then stages from q and dO).
  uint32_t* xq;
  uint32_t* xd;
  // bf16 with G >= 2: per query-pass workgroup ([B][Hkv][n / bq]), a bound
  // on |dS| / scale over its (query, head, slot) entries, from which the key
  // pass scales its f16 dS weights by a power of two.  Null otherwise.
  float* wmax;
  size_t bytes;
  int blocks;
};
size_t bwd_workspace_layout(const Problem& p, const SlotTable& t, void* base,
                            BwdWorkspace* ws);

// Edge-list backward: workspace p, dp [B*Hkv][n][width][G], Dvec / l and
// 1 / l [B*Hkv][n][G] (floats; l = sum over the list of p); returns its size
// in bytes.
size_t bwd_edges_workspace_layout(const Problem& p, int width, void* base, float** P, float** dP,
                                  float** Dvec, float** Linv);
int launch_bwd_edges(const Problem& p, const int32_t* edges, const int32_t* count, int width,
                     const int32_t* inv, const int32_t* inv_count, int inv_width, const void* q,
                     const void* k, const void* v, const float* lse, const void* dout, void* dq,
                     void* dk, void* dv, void* workspace, void* stream);

int launch_bwd_query(const Problem& p, const SlotTable& t, const void* q,
                     const void* k, const void* v, const float* lse,
                     const void* dout, void* dq, const BwdWorkspace& ws,
                     bool want_dd, void* stream);
// With dd or dtheta requested the bf16 key pass also reduces them (see
// bwd_key_reduces); otherwise base_f, alpha, dd and dtheta are unused.
int launch_bwd_key(const Problem& p, const SlotTable& t, const void* q,
                   const void* k, const void* v, const void* dout, void* dk,
                   void* dv, const BwdWorkspace& ws, const float* base_f,
                   double alpha, float* dd, float* dtheta, void* stream);
// Whether launch_bwd_key reduces dd / dtheta itself (want: either is asked).
bool bwd_key_reduces(const Problem& p, const SlotTable& t, bool want);
int launch_bwd_reduce(const SlotTable& t, const BwdWorkspace& ws,
                      const float* base_f, double alpha, float* dd,
                      float* dtheta, void* stream);

// sfa_bwd's validation and launches with the workspace given; shared by the
// entry points that bring their own workspace and the one that uses the
// library's static scratch (fn names the caller in error messages).
int bwd_impl(const sfa_attn* a, const void* q, const void* k, const void* v, const float* lse, const void* dout,
             void* dq, void* dk, void* dv, float* dd, const int32_t* base, double alpha, float* dtheta,
             void* workspace, size_t ws_bytes, void* stream, const char* fn);
// Workspace bytes sfa_bwd needs (0 after recording the error on bad input).
size_t bwd_workspace_bytes(const sfa_attn* a);

// Event-pair bracketing for sfa_profile_*; no-ops while profiling is off.
// While a scope records, the first launch inside it (through SFA_LAUNCH)
// takes the pair as the dispatch's own start and end timestamps
// (hipExtLaunchKernelGGL), so no event packets enter the stream to hold
// back the next kernel.  A scope with more launches re-records its end
// event after the last one; a scope without a launch records nothing.
struct ProfileScope {
  ProfileScope(const char* name, void* stream);
  ~ProfileScope();
  const char* name;
  void* stream;
  void* ev0;
  void* ev1;
  int launches;  // launches made through SFA_LAUNCH inside the scope
};

// The recording scope of this thread, or null.
ProfileScope* active_profile_scope();

}  // namespace sfa
