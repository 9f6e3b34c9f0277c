// Host-side validation of a block index (prism_check_index).
//
// The attention entry points read the permutation, the block starts and the
// two block lists on the device without checking their contents; a caller
// that builds or edits an index itself checks a host copy here first.  The
// rules are the invariants the pages' partition and selection give every
// index (Prism pt reading guide, Método 2 and 3: each 8x8x8 zone is cut into
// equal blocks of 64, 128 or 256 tokens, every query block attends to a
// non-empty set S_i of key blocks), plus the layout prism_select_blocks
// writes.

#include <stdint.h>
#include <string.h>

#include <vector>

#include "../../include/prism.h"

namespace {

struct Bad {
  int64_t* out;
  int fail(int64_t head, int64_t item) {
    if (out) {
      out[0] = head;
      out[1] = item;
    }
    return PRISM_EINDEX;
  }
};

// One list array laid out as prism_select_blocks writes it: [heads][tiles + 1]
// pointers with offsets counted over all heads, lists of ascending block
// indices below nb.  nonempty: every list must hold at least one entry.
// Returns the status; *end receives the head's end offset.
int check_lists(const int32_t* ptr, const int32_t* idx, int64_t tiles, int32_t nb, int64_t base, int64_t n_idx,
                bool nonempty, int64_t head, int64_t item_base, Bad& bad, int64_t* end) {
  if (ptr[0] != base) return bad.fail(head, item_base);
  for (int64_t b = 0; b < nb; ++b) {
    const int64_t lo = ptr[b], hi = ptr[b + 1];
    if (hi < lo || hi > n_idx) return bad.fail(head, item_base + b);
    if (nonempty && hi == lo) return bad.fail(head, item_base + b);
    for (int64_t e = lo; e < hi; ++e) {
      if (idx[e] < 0 || idx[e] >= nb) return bad.fail(head, item_base + b);
      if (e > lo && idx[e] <= idx[e - 1]) return bad.fail(head, item_base + b);
    }
  }
  for (int64_t b = nb + 1; b <= tiles; ++b)
    if (ptr[b] != ptr[nb]) return bad.fail(head, item_base + b);
  *end = ptr[nb];
  return PRISM_OK;
}

}  // namespace

extern "C" int prism_check_index(const prism_problem* prob, const int32_t* perm, const int32_t* blk_start,
                                 const int32_t* n_blocks, const int32_t* row_ptr, const int32_t* col_idx,
                                 const int32_t* t_row_ptr, const int32_t* t_col_idx, int64_t n_idx, int64_t* bad_out) {
  if (!prob || !blk_start || !n_blocks || !row_ptr || !col_idx || n_idx < 0) return PRISM_EINVAL;
  if ((t_row_ptr == nullptr) != (t_col_idx == nullptr)) return PRISM_EINVAL;
  if (prob->T <= 0 || prob->H <= 0 || prob->W <= 0 || prob->T % 8 || prob->H % 8 || prob->W % 8) return PRISM_EGRID;
  if (prob->heads < 1) return PRISM_EINVAL;
  Bad bad{bad_out};
  if (bad_out) bad_out[0] = bad_out[1] = -1;
  const int64_t N = (int64_t)prob->T * prob->H * prob->W;
  const int64_t tiles = N / 64;
  std::vector<uint8_t> seen(perm ? (size_t)N : 0);
  std::vector<int32_t> count;
  int64_t base = 0, tbase = 0;
  for (int64_t h = 0; h < prob->heads; ++h) {
    // block starts: item numbers 0 .. tiles
    const int32_t nb = n_blocks[h];
    const int32_t* bs = blk_start + h * (tiles + 1);
    if (nb < tiles / 4 || nb > tiles) return bad.fail(h, -1);
    if (bs[0] != 0) return bad.fail(h, 0);
    for (int32_t b = 0; b < nb; ++b) {
      const int32_t s = bs[b], e = bs[b + 1], n = e - s;
      if (n != 1 && n != 2 && n != 4) return bad.fail(h, b);
      if (s % n != 0 || s / 8 != (e - 1) / 8) return bad.fail(h, b);   // equal blocks inside one zone
    }
    for (int64_t b = nb; b <= tiles; ++b)
      if (bs[b] != tiles) return bad.fail(h, b);
    // permutation: a bijection of the head's tokens (item = position)
    if (perm) {
      memset(seen.data(), 0, seen.size());
      const int32_t* p = perm + h * N;
      for (int64_t i = 0; i < N; ++i) {
        if (p[i] < 0 || p[i] >= N || seen[p[i]]) return bad.fail(h, i);
        seen[p[i]] = 1;
      }
    }
    // query-major lists (item = query block): non-empty, ascending, below nb
    int64_t end = 0;
    int st = check_lists(row_ptr + h * (tiles + 1), col_idx, tiles, nb, base, n_idx, true, h, 0, bad, &end);
    if (st != PRISM_OK) return st;
    // key-major lists (items numbered from tiles + 1): the exact transpose
    if (t_row_ptr) {
      int64_t tend = 0;
      st = check_lists(t_row_ptr + h * (tiles + 1), t_col_idx, tiles, nb, tbase, n_idx, false, h, tiles + 1, bad,
                       &tend);
      if (st != PRISM_OK) return st;
      if (tend - tbase != end - base) return bad.fail(h, tiles + 1);
      const int32_t* rp = row_ptr + h * (tiles + 1);
      const int32_t* tp = t_row_ptr + h * (tiles + 1);
      count.assign((size_t)nb, 0);
      for (int32_t i = 0; i < nb; ++i)      // rows ascending: each column's rows arrive in order
        for (int64_t e = rp[i]; e < rp[i + 1]; ++e) {
          const int32_t j = col_idx[e];
          const int64_t at = tp[j] + count[j];
          if (at >= tp[j + 1] || t_col_idx[at] != i) return bad.fail(h, tiles + 1 + j);
          ++count[j];
        }
      for (int32_t j = 0; j < nb; ++j)
        if (tp[j] + count[j] != tp[j + 1]) return bad.fail(h, tiles + 1 + j);
      tbase = tend;
    }
    base = end;
  }
  return PRISM_OK;
}
