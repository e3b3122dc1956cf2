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

// Where the requests' tokens and entries are, and which entries each token
// sees.  A null qo (kvp) stands for the single range [0, T) ([0, kv_cap)): one
// request holding every token (entry).
//
// Causal draft tokens see a prefix of their request's entry list: token j of
// qlen sees the entries at global positions <= N - qlen + j, N being the
// request's total entry count.  Without context parallelism (gkvp null) the
// list holds every position in order, so token j sees n - (qlen - 1 - j) of
// its n entries.  Under DCP the positions are dealt round-robin over cp_size
// shards: this shard (cp_rank) holds positions cp_rank + i * cp_size, i = 0..,
// gkvp gives N per request, and token j sees the local entries i with
// cp_rank + i * cp_size <= N - qlen + j ("Kimi K3 on AMD Instinct MI355X ...",
// Sec. 1: each GPU keeps an eighth of the positions; multi-token verification
// under DCP).
//
// Paged caches (page_size = 2^page_shift > 1): kvp counts pages, kv_indices
// holds page (block) numbers, and request b's last page holds lpl[b] of its
// page_size slots, so it has (pages - 1) * page_size + lpl[b] entries.
struct ReqSource {
  const int32_t* qo;    // (B+1) query-token offsets, or null
  const int32_t* kvp;   // (B+1) local entry (page) offsets, or null
  const int32_t* gkvp;  // (B+1) offsets of the requests' full (all-shard) lists, or null
  int kv_cap;           // entries (pages) in kv_indices
  int T;                // query tokens
  int causal;           // 0: every token sees all of its request's local entries
  int cp_size;          // shards the positions are dealt over (1 without DCP)
  int cp_rank;          // this shard
  const int32_t* lpl;   // (B) used slots of each request's last page (paged caches)
  int page_shift;       // log2(page_size); 0: one entry per index
  // Shared-prefix (cascade) view, on when prefix_len >= 0: the caller's B
  // requests become B + 1 over 2T tokens.  Request 0 is every token (tokens
  // 0 .. T-1) against entries [0, prefix_len), all visible; request b + 1 is
  // request b's tokens (T + qo[b] ..) against its own entries prefix_len +
  // kvp[b] .., under `causal`.  qo / kvp are then the caller's qo_indptr and
  // suffix offsets, and T above is the ReqSource's T / 2.
  int prefix_len;
};

// One request's bounds, clamped so that no later read can leave its buffer,
// and its visibility rule: token j sees min(n, (vbase + j) / vstep + 1)
// entries when vbase + j >= 0, none otherwise.
struct Req {
  int kv_base;  // offset of its first entry (page) in kv_indices
  int n;        // local entry count
  int q_base;   // its first query token
  int qlen;     // query tokens
  int causal;   // 0: every token sees all n
  int vbase;    // N - qlen - cp_rank
  int vstep;    // cp_size
};

MLA_HD Req load_req(const ReqSource& s, int b) {
  int k0, k1, q0, q1, causal = s.causal;
  if (s.prefix_len >= 0) {  // cascade view
    const int T = s.T / 2, P = imin(s.prefix_len, s.kv_cap);
    if (b == 0) {
      k0 = 0;
      k1 = P;
      q0 = 0;
      q1 = T;
      causal = 0;
    } else {
      k0 = imax(P + s.kvp[b - 1], P);
      k1 = P + s.kvp[b];
      q0 = imax(T + s.qo[b - 1], T);
      q1 = T + s.qo[b];
    }
  } else {
    k0 = s.kvp ? s.kvp[b] : 0;
    k1 = s.kvp ? s.kvp[b + 1] : s.kv_cap;
    q0 = s.qo ? s.qo[b] : 0;
    q1 = s.qo ? s.qo[b + 1] : s.T;
  }
  k0 = imin(imax(k0, 0), s.kv_cap);
  k1 = imin(imax(k1, k0), s.kv_cap);
  q0 = imin(imax(q0, 0), s.T);
  q1 = imin(imax(q1, q0), s.T);
  Req r;
  r.kv_base = k0;
  r.n = k1 - k0;
  if (s.page_shift > 0 && r.n > 0) {
    const int P = 1 << s.page_shift;
    r.n = ((r.n - 1) << s.page_shift) + imin(imax(s.lpl[b], 1), P);
  }
  r.q_base = q0;
  r.qlen = q1 - q0;
  r.causal = causal;
  if (s.gkvp) {
    const int N = imax(s.gkvp[b + 1] - s.gkvp[b], 0);
    r.vbase = N - r.qlen - s.cp_rank;
    r.vstep = imax(s.cp_size, 1);
  } else {
    r.vbase = r.n - r.qlen;
    r.vstep = 1;
  }
  return r;
}

// Entries visible to token j of request r (never decreasing in j).
MLA_HD int req_visible(const Req& r, int j) {
  if (!r.causal) return r.n;
  const int x = r.vbase + j;
  return x < 0 ? 0 : imin(r.n, x / r.vstep + 1);
}

// First token of r with a non-empty visible set (qlen if none): the number of
// tokens of r that see nothing.
MLA_HD int first_visible_token(const Req& r) {
  if (r.n == 0) return r.qlen;
  return r.causal ? imin(r.qlen, imax(0, -r.vbase)) : 0;
}

MLA_HD int req_empty_tokens(const Req& r) { return first_visible_token(r); }

// Sum over the request's query tokens of their visible entries.
MLA_HD int64_t request_rows(const Req& r) {
  int64_t s = 0;
  for (int j = first_visible_token(r); j < r.qlen; ++j) s += req_visible(r, j);
  return s;
}

// Position in the unit stream: request b, its token j, head group g, offset k.
struct Cursor {
  int b, j, g, k;
  Req r;
};

// Place the cursor at offset `off` (< G * request_rows) inside request b.
MLA_HD void cursor_in_request(Cursor& c, int b, const Req& r, int64_t off, int G) {
  c.b = b;
  c.r = r;
  for (int j = first_visible_token(r); j < r.qlen; ++j) {
    const int v = req_visible(r, j);
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
  return snap_position(x, c.k, req_visible(c.r, c.j));
}

// Move to the start of the next non-empty unit.  Returns false past the end.
MLA_HD bool cursor_next_unit(Cursor& c, const ReqSource& src, int B, int G) {
  c.k = 0;
  if (++c.g < G) return true;
  c.g = 0;
  ++c.j;
  if (c.j < c.r.qlen) return true;  // visible counts never decrease with j
  for (int b = c.b + 1; b < B; ++b) {
    const Req r = load_req(src, b);
    if (request_rows(r) > 0) {
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
// row groups).  The request's query rows (token j, head h), qlen * H of them,
// are numbered j * H + h and cut into row groups of 16 (the last may be
// partial): with H a multiple of 16, row group rg is token rg / G, head group
// rg % G; with any other H (12 real heads, unpadded) a row group may hold rows
// of two or more tokens, and no MFMA row is spent on padding.  Unit u covers
// row groups [8u, 8u + 8) and is as long as its last row sees (the other rows
// mask the entries they may not see).  Used when
// a request may hold four or more row groups (many heads or several query
// tokens), where a unit per row group would gather the same rows once per row
// group; a unit with fewer than eight leaves some MFMA rows idle, which costs
// less than the repeated gathers.
constexpr int kGroupsPerUnit = 8;
constexpr int kGroupModeMinRows = 4;

// Partial-answer slots per worker: a worker holds at most two partial pieces,
// each covering one row group, or kGroupsPerUnit row groups in group mode.
MLA_HD int slots_per_worker(bool group_mode) { return group_mode ? 2 * kGroupsPerUnit : 2; }

MLA_HD bool use_group_mode(int G, int max_seqlen_q) {
  return (int64_t)G * max_seqlen_q >= kGroupModeMinRows;
}

// Row groups of request r with H heads per token.
MLA_HD int group_row_groups(const Req& r, int H) { return (r.qlen * H + kGroup - 1) / kGroup; }

// Row-group entries per query token in the descriptor layout: request r's
// row group rg has entry q_base * group_slots_per_token(H) + rg (a request's
// ceil(qlen * H / 16) row groups never exceed its tokens' qlen * ceil(H / 16)
// entries; entries past them are unused).
MLA_HD int group_slots_per_token(int H) { return (H + kGroup - 1) / kGroup; }

MLA_HD int group_units(const Req& r, int H) {
  return (group_row_groups(r, H) + kGroupsPerUnit - 1) / kGroupsPerUnit;
}

// Token of the last row of row group rg.
MLA_HD int group_last_token(const Req& r, int H, int rg) {
  return imin(kGroup * rg + kGroup - 1, r.qlen * H - 1) / H;
}

MLA_HD int group_unit_len(const Req& r, int H, int u) {
  const int last = imin(kGroupsPerUnit * u + kGroupsPerUnit - 1, group_row_groups(r, H) - 1);
  return req_visible(r, group_last_token(r, H, last));
}

// A group-mode piece has fixed work worth about kGroupPieceRows rows of its
// tile loop (q and index staging, the first tile loads, the last pair's P.V,
// eight row groups of partial stores), so in the work stream every non-empty
// unit is that many rows longer than its entries: its span.  The extra rows come first, so the
// worker whose share takes in a unit's start is charged for starting it; a
// share boundary inside those rows hands the whole start to the later worker
// (the earlier one then holds no piece of the unit).  With equal shares of
// spans, a worker that holds two pieces gets correspondingly fewer entries.
// (Timestamps per workgroup put a second piece at ~38K cycles, ~10 tiles.)
constexpr int kGroupPieceRows = 320;

MLA_HD int group_unit_span(const Req& r, int H, int u) {
  const int v = group_unit_len(r, H, u);
  return v > 0 ? v + kGroupPieceRows : 0;
}

// Stream rows of request r in group mode (the sum of its units' spans).
MLA_HD int64_t group_request_rows(const Req& r, int H) {
  int64_t s = 0;
  const int U = group_units(r, H);
  for (int u = 0; u < U; ++u) s += group_unit_span(r, H, u);
  return s;
}

// Position in the group-mode stream: request b, its unit u, offset k within
// the unit's span (entry k - kGroupPieceRows, or the unit's start before it).
struct GCursor {
  int b, u, k;
  Req r;
};

MLA_HD void gcursor_in_request(GCursor& c, int b, const Req& r, int64_t off, int H) {
  c.b = b;
  c.r = r;
  const int U = group_units(r, H);
  for (int u = 0; u < U; ++u) {
    const int v = group_unit_span(r, H, u);
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

// The entries [k0, k0 + len) of its unit that the stream rows [k, k + n) of a
// span cover (len may be 0: rows that only charge the unit's start).
MLA_HD void group_piece_entries(int k, int n, int& k0, int& len) {
  k0 = imax(k - kGroupPieceRows, 0);
  len = imax(k + n - kGroupPieceRows, 0) - k0;
}

// Move to the start of the next non-empty unit (unit lengths never shrink
// within a request).  Returns false past the end.
MLA_HD bool gcursor_next_unit(GCursor& c, const ReqSource& src, int B, int H) {
  c.k = 0;
  if (++c.u < group_units(c.r, H)) return true;
  for (int b = c.b + 1; b < B; ++b) {
    const Req r = load_req(src, b);
    if (group_request_rows(r, H) > 0) {
      c.b = b;
      c.r = r;
      c.u = 0;
      while (group_unit_len(r, H, c.u) == 0) ++c.u;
      return true;
    }
  }
  return false;
}

MLA_HD int64_t gsnap_at(int64_t x, const GCursor& c, int H) {
  return snap_position(x, c.k, group_unit_span(c.r, H, c.u));
}

}  // namespace mla
