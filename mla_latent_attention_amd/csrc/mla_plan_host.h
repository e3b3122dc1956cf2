// mla_plan_host.h - host mirror of the device planners (plain C++, no HIP).
//
// Walks the same equal-share, boundary-snapped plan the decode kernels derive
// on the device (mla_plan.h) and lists every worker's pieces (group mode:
// their entries, not the stream rows that charge a unit's start), for the
// tests:
// the C ABI exports it as mla_plan_host / mla_plan_groups_host, and a
// sanitizer build of the tests includes it directly.
#pragma once

#include <stdint.h>

#include <vector>

#include "mla_plan.h"

namespace mla {

inline int64_t plan_pieces_host(const int32_t* qo_indptr, const int32_t* kv_indptr,
                                const int32_t* g_kv_indptr, int batch, int num_heads,
                                int num_workers, int cp_world_size, int cp_rank, int64_t* out,
                                int64_t out_cap) {
  if (!qo_indptr || !kv_indptr || batch < 1 || num_heads < kGroup || num_heads % kGroup ||
      num_workers < 1 || (out_cap > 0 && !out))
    return -1;
  if (cp_world_size < 1 || cp_rank < 0 || cp_rank >= cp_world_size) return -1;
  const int G = num_heads / kGroup;
  const int T = qo_indptr[batch];
  const int kv_cap = kv_indptr[batch];
  if (T < 0 || kv_cap < 0) return -1;
  const ReqSource src{qo_indptr, kv_indptr, g_kv_indptr, kv_cap, T, 1, cp_world_size, cp_rank,
                      nullptr, 0, -1};
  std::vector<int64_t> cum(batch + 1, 0);
  for (int b = 0; b < batch; ++b) cum[b + 1] = cum[b] + (int64_t)G * request_rows(load_req(src, b));
  const int64_t W = cum[batch];
  if (W == 0) return 0;
  const int nw = effective_workers(W, num_workers);
  int64_t count = 0;
  // Cursor at stream position x (0 <= x < W), as the kernel's locate does.
  auto locate = [&](int64_t x, Cursor& c) {
    int b = 0;
    while (!(cum[b] <= x && x < cum[b + 1])) ++b;
    cursor_in_request(c, b, load_req(src, b), x - cum[b], G);
  };
  for (int w = 0; w < nw; ++w) {
    const int64_t x0 = worker_begin(w, W, nw), x1 = worker_begin(w + 1, W, nw);
    Cursor c, c1;
    locate(x0, c);
    int64_t p1 = W;
    if (x1 < W) {
      locate(x1, c1);
      p1 = snap_at(x1, c1);
    }
    const int64_t p0 = snap_at(x0, c);
    if (p0 >= p1) continue;
    if (p0 < x0) {
      c.k = 0;
    } else if (p0 > x0) {
      if (!cursor_next_unit(c, src, batch, G)) continue;
    }
    int64_t pos = p0;
    int piece = 0;
    while (pos < p1) {
      const int v = req_visible(c.r, c.j);
      const int len = (int)lmin((int64_t)(v - c.k), p1 - pos);
      if (len <= 0) return -1;
      const bool complete = (c.k == 0 && len == v);
      const int slot = complete ? -1 : (piece == 0 ? 2 * w : 2 * w + 1);
      if (count < out_cap) {
        int64_t* rec = out + 8 * count;
        rec[0] = w;
        rec[1] = c.r.q_base + c.j;
        rec[2] = c.g;
        rec[3] = c.k;
        rec[4] = c.k + len;
        rec[5] = v;
        rec[6] = slot;
        rec[7] = complete ? 1 : 0;
      }
      ++count;
      pos += len;
      c.k += len;
      ++piece;
      if (pos < p1 && c.k == v && !cursor_next_unit(c, src, batch, G))
        return -1;
    }
  }
  return count;
}

inline int64_t plan_group_pieces_host(const int32_t* qo_indptr, const int32_t* kv_indptr,
                                      const int32_t* g_kv_indptr, int batch, int num_heads,
                                      int num_workers, int causal, int cp_world_size,
                                      int cp_rank, int64_t* out, int64_t out_cap) {
  if (!qo_indptr || !kv_indptr || batch < 1 || num_heads < 1 || num_workers < 1 ||
      (out_cap > 0 && !out))
    return -1;
  if (cp_world_size < 1 || cp_rank < 0 || cp_rank >= cp_world_size) return -1;
  const int H = num_heads;  // any count: rows are packed 16 to a row group
  const int T = qo_indptr[batch];
  const int kv_cap = kv_indptr[batch];
  if (T < 0 || kv_cap < 0) return -1;
  const ReqSource src{qo_indptr, kv_indptr, g_kv_indptr, kv_cap, T, causal ? 1 : 0, cp_world_size,
                      cp_rank, nullptr, 0, -1};
  std::vector<int64_t> cum(batch + 1, 0);
  for (int b = 0; b < batch; ++b) cum[b + 1] = cum[b] + group_request_rows(load_req(src, b), H);
  const int64_t W = cum[batch];
  if (W == 0) return 0;
  const int nw = effective_workers(W, num_workers);
  const int slots = slots_per_worker(true);
  int64_t count = 0;
  auto locate = [&](int64_t x, GCursor& c) {
    int b = 0;
    while (!(cum[b] <= x && x < cum[b + 1])) ++b;
    gcursor_in_request(c, b, load_req(src, b), x - cum[b], H);
  };
  for (int w = 0; w < nw; ++w) {
    const int64_t x0 = worker_begin(w, W, nw), x1 = worker_begin(w + 1, W, nw);
    GCursor c, c1;
    locate(x0, c);
    int64_t p1 = W;
    if (x1 < W) {
      locate(x1, c1);
      p1 = gsnap_at(x1, c1, H);
    }
    const int64_t p0 = gsnap_at(x0, c, H);
    if (p0 >= p1) continue;
    if (p0 < x0) {
      c.k = 0;
    } else if (p0 > x0) {
      if (!gcursor_next_unit(c, src, batch, H)) continue;
    }
    int64_t pos = p0;
    int piece = 0;
    while (pos < p1) {
      const int L = group_unit_len(c.r, H, c.u);
      const int span = L + kGroupPieceRows;
      const int n = (int)lmin((int64_t)(span - c.k), p1 - pos);
      if (n <= 0) return -1;
      int k0, len;
      group_piece_entries(c.k, n, k0, len);
      if (len > 0) {
        const bool complete = (k0 == 0 && len == L);
        const int slot = complete ? -1 : slots * w + (piece == 0 ? 0 : slots / 2);
        if (count < out_cap) {
          int64_t* rec = out + 8 * count;
          rec[0] = w;
          rec[1] = c.b;
          rec[2] = c.u;
          rec[3] = k0;
          rec[4] = k0 + len;
          rec[5] = L;
          rec[6] = slot;
          rec[7] = complete ? 1 : 0;
        }
        ++count;
        ++piece;
      }
      pos += n;
      c.k += n;
      if (pos < p1 && c.k == span && !gcursor_next_unit(c, src, batch, H))
        return -1;
    }
  }
  return count;
}

}  // namespace mla
