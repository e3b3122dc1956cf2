// mla_plan.h - work planner shared by the decode kernel, the split combine
// kernel and the host mirror (mla_plan_host).
//
// The pages attribute the long-context decode win to dividing a request's KV
// history into pieces processed by separate workgroups and combining the
// results ("Kimi K3 on AMD Instinct MI355X: vLLM Serving Matches NVIDIA HGX
// B300 Throughput per GPU on AgentX", Sec. 4 "MLA: faster long-context
// decoding with AMD AITER assembly").  This planner is our own:
//
//   * A "unit" is one (query token t, group of 16 heads g); its length is the
//     number of KV entries token t may see (all of its request's entries for
//     single-token decode; bottom-right causal for several query tokens).
//   * Units are laid end to end in (request, token, head group) order, giving
//     a stream of W = sum of unit lengths KV rows.
//   * Worker w (one workgroup) takes stream positions
//     [floor(w*W/NW), floor((w+1)*W/NW)), so every worker gets the same number
//     of KV rows (+-1) whatever the length mix; the range may cross unit and
//     request boundaries.  The part of a unit inside one worker is a "piece".
//   * A worker boundary that falls within kSnapRows rows of a unit boundary
//     is moved onto it, so no worker pays the fixed cost of a piece of a few
//     rows (with equal shares, unit boundaries drift a few rows past worker
//     boundaries).  Unsnapped boundaries are >= kMinWorkerRows - 1 rows apart
//     and each moves at most kSnapRows, so they never meet.
//   * Only a worker's first and last piece can be partial: a partial first
//     piece writes its (o, lse) to workspace slot 2w, a partial last piece to
//     slot 2w+1.  Complete pieces write o (and lse) directly.
//   * NW is capped so that every worker gets at least kMinWorkerRows rows.
//
// Everything is computed from qo_indptr / kv_indptr on the device, so a call
// needs no metadata kernel and no host synchronisation.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define MLA_HD __host__ __device__ __forceinline__
#else
#define MLA_HD inline
#endif

namespace mla {

constexpr int kRowDim = 576;     // latent 512 + rope 64
constexpr int kLatent = 512;
constexpr int kGroup = 16;       // heads per row group (one MFMA tile of rows)
constexpr int kMinWorkerRows = 256;

MLA_HD int imin(int a, int b) { return a < b ? a : b; }
MLA_HD int imax(int a, int b) { return a > b ? a : b; }
MLA_HD int64_t lmin(int64_t a, int64_t b) { return a < b ? a : b; }

// Entries visible to query token j of a request with qlen tokens and n entries.
MLA_HD int visible(int n, int qlen, int j) { return imax(0, n - (qlen - 1 - j)); }

// Sum over the request's query tokens of their visible entries.
MLA_HD int64_t request_rows(int n, int qlen) {
  int m = imin(qlen, n);
  if (m <= 0) return 0;
  return (int64_t)m * n - (int64_t)m * (m - 1) / 2;
}

MLA_HD int effective_workers(int64_t W, int nw) {
  int64_t need = W / kMinWorkerRows;  // rounded down: every worker gets >= kMinWorkerRows
  if (need < 1) need = 1;
  return (int)lmin(need, (int64_t)nw);
}

// Unsnapped start of worker w's range.
MLA_HD int64_t worker_begin(int w, int64_t W, int nw) { return (int64_t)w * W / nw; }

constexpr int kSnapRows = 64;

// Snapped position for stream position x lying k rows into a unit of length
// v: the nearer unit boundary if it is within kSnapRows rows, else x.
MLA_HD int64_t snap_position(int64_t x, int k, int v) {
  if (k == 0) return x;
  if (k <= kSnapRows && k <= v - k) return x - k;
  if (v - k <= kSnapRows) return x + (v - k);
  return x;
}

// One request's bounds, clamped so that no later read can leave its buffer.
struct Req {
  int kv_base;  // offset of its first entry in kv_indices
  int n;        // KV length
  int q_base;   // its first query token
  int qlen;     // query tokens
  int causal;   // 1: token j sees visible(n, qlen, j) entries; 0: every token sees all n
};

// Request b's bounds.  A null qo (kvp) stands for the single range [0, T)
// ([0, kv_cap)): one request holding every token (entry).
MLA_HD Req load_req(const int32_t* qo, const int32_t* kvp, int b, int kv_cap, int T,
                    int causal = 1) {
  int k0 = kvp ? kvp[b] : 0, k1 = kvp ? kvp[b + 1] : kv_cap;
  int q0 = qo ? qo[b] : 0, q1 = qo ? qo[b + 1] : T;
  k0 = imin(imax(k0, 0), kv_cap);
  k1 = imin(imax(k1, k0), kv_cap);
  q0 = imin(imax(q0, 0), T);
  q1 = imin(imax(q1, q0), T);
  Req r;
  r.kv_base = k0;
  r.n = k1 - k0;
  r.q_base = q0;
  r.qlen = q1 - q0;
  r.causal = causal;
  return r;
}

// Entries visible to token j of request r.
MLA_HD int req_visible(const Req& r, int j) { return r.causal ? visible(r.n, r.qlen, j) : r.n; }

// Tokens of r that see no entry.
MLA_HD int req_empty_tokens(const Req& r) {
  return r.causal ? imin(r.qlen, imax(0, r.qlen - r.n)) : (r.n == 0 ? r.qlen : 0);
}

// Position in the unit stream: request b, its token j, head group g, offset k.
struct Cursor {
  int b, j, g, k;
  Req r;
};

// First token of r with a non-empty visible set.
MLA_HD int first_visible_token(const Req& r) { return imax(0, r.qlen - r.n); }

// Place the cursor at offset `off` (< G * request_rows) inside request b.
MLA_HD void cursor_in_request(Cursor& c, int b, const Req& r, int64_t off, int G) {
  c.b = b;
  c.r = r;
  for (int j = first_visible_token(r); j < r.qlen; ++j) {
    int v = visible(r.n, r.qlen, j);
    int64_t rows = (int64_t)G * v;
    if (off < rows) {
      c.j = j;
      c.g = (int)(off / v);
      c.k = (int)(off % v);
      return;
    }
    off -= rows;
  }
  c.j = r.qlen;  // not reached for a valid offset
  c.g = 0;
  c.k = 0;
}

// Snap stream position x whose cursor is c (set by cursor_in_request).
MLA_HD int64_t snap_at(int64_t x, const Cursor& c) {
  return snap_position(x, c.k, visible(c.r.n, c.r.qlen, c.j));
}

// Move to the start of the next non-empty unit.  Returns false past the end.
MLA_HD bool cursor_next_unit(Cursor& c, const int32_t* qo, const int32_t* kvp, int B, int kv_cap,
                             int T, int G) {
  c.k = 0;
  if (++c.g < G) return true;
  c.g = 0;
  ++c.j;
  if (c.j < c.r.qlen) return true;  // visible counts only grow with j
  for (int b = c.b + 1; b < B; ++b) {
    Req r = load_req(qo, kvp, b, kv_cap, T);
    if (request_rows(r.n, r.qlen) > 0) {
      c.b = b;
      c.r = r;
      c.j = first_visible_token(r);
      return true;
    }
  }
  return false;
}

// ---- Group mode: a unit is kGroupsPerUnit consecutive row groups of one
// request, processed by one workgroup over one shared KV range (each wave two
// row groups).  Row group rg = j * G + g (token j, head group g); unit u covers
// row groups [8u, 8u + 8) of the request's qlen * G and is as long as the
// last of them sees (the others mask the entries they may not see).  Used when
// a request may hold four or more row groups (many heads or several query
// tokens), where a unit per row group would gather the same rows once per row
// group; a unit with fewer than eight leaves some MFMA rows idle, which costs
// less than the repeated gathers.
constexpr int kGroupsPerUnit = 8;
constexpr int kGroupModeMinRows = 4;

MLA_HD bool use_group_mode(int G, int max_seqlen_q) {
  return (int64_t)G * max_seqlen_q >= kGroupModeMinRows;
}

MLA_HD int group_units(const Req& r, int G) {
  return (r.qlen * G + kGroupsPerUnit - 1) / kGroupsPerUnit;
}

MLA_HD int group_unit_len(const Req& r, int G, int u) {
  const int last = imin(kGroupsPerUnit * u + kGroupsPerUnit - 1, r.qlen * G - 1);
  return req_visible(r, last / G);
}

// Stream rows of request r in group mode.
MLA_HD int64_t group_request_rows(const Req& r, int G) {
  int64_t s = 0;
  const int U = group_units(r, G);
  for (int u = 0; u < U; ++u) s += group_unit_len(r, G, u);
  return s;
}

// Position in the group-mode stream: request b, its unit u, offset k.
struct GCursor {
  int b, u, k;
  Req r;
};

MLA_HD void gcursor_in_request(GCursor& c, int b, const Req& r, int64_t off, int G) {
  c.b = b;
  c.r = r;
  const int U = group_units(r, G);
  for (int u = 0; u < U; ++u) {
    const int v = group_unit_len(r, G, u);
    if (off < v) {
      c.u = u;
      c.k = (int)off;
      return;
    }
    off -= v;
  }
  c.u = U;  // not reached for a valid offset
  c.k = 0;
}

// Move to the start of the next non-empty unit (unit lengths never shrink
// within a request).  Returns false past the end.
MLA_HD bool gcursor_next_unit(GCursor& c, const int32_t* qo, const int32_t* kvp, int B, int kv_cap,
                              int T, int G, int causal) {
  c.k = 0;
  if (++c.u < group_units(c.r, G)) return true;
  for (int b = c.b + 1; b < B; ++b) {
    Req r = load_req(qo, kvp, b, kv_cap, T, causal);
    if (group_request_rows(r, G) > 0) {
      c.b = b;
      c.r = r;
      c.u = 0;
      while (group_unit_len(r, G, c.u) == 0) ++c.u;
      return true;
    }
  }
  return false;
}

MLA_HD int64_t gsnap_at(int64_t x, const GCursor& c, int G) {
  return snap_position(x, c.k, group_unit_len(c.r, G, c.u));
}

}  // namespace mla
