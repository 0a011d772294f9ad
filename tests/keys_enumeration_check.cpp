// CPU check of the key-major work-item enumeration of the attention backward and the
// indexer-key gradients (long_context_compressed_amd/csrc/attn_bwd_keys.h): the helpers that
// the device planner (k_attn_bwd_keys_plan) and the host capacity bound share.  For random
// packed batches, query chunks, ratios, windows and modes it enumerates the items the way the
// planner does (per sample: compressed blocks by query chunk, then window blocks), gives
// every item a partial slot and every block a reduction record, and checks that
//   * every (query, visible compressed row) and (query, window row) pair of the chunk is in
//     exactly one item, and no item reaches outside its sample or chunk;
//   * items, partial slots and records stay within item_cap;
//   * each record's slots are exactly the items of its block.
// Prints "pairs <n> failures <f>"; exit status 1 on any failure.
#include <algorithm>
#include <cstdio>
#include <map>
#include <random>
#include <vector>

#include "../long_context_compressed_amd/csrc/attn_bwd_keys.h"

using namespace csa::keys;

namespace {

struct Item {
  int key0, nk, kind, q0, nq, part;
};
struct Record {
  int key0, nk, kind, first, count;
};

int run(int kb, int trials, unsigned seed, long long* pairs) {
  std::mt19937 rng(seed);
  int fails = 0;
  auto fail = [&](const char* what) {
    if (fails < 10) std::printf("kb %d: %s\n", kb, what);
    ++fails;
  };
  for (int trial = 0; trial < trials; ++trial) {
    const int B = 1 + rng() % 5, r = (rng() % 3 == 0) ? 128 : 4, W = 1 + rng() % 200;
    const int mode = rng() % 3;   // 0 selected rows, 1 dense, 2 window only
    std::vector<int> L(B);
    int T = 0, max_len = 1;
    for (int b = 0; b < B; ++b) {
      L[b] = (rng() % 5 == 0) ? rng() % 20 : rng() % 2600;
      T += L[b];
      max_len = std::max(max_len, L[b]);
    }
    if (T == 0) continue;
    int n_cap = max_len / r;
    if (rng() % 4 == 0) n_cap = std::max(1, n_cap / 2);
    std::vector<int> cu(B + 1, 0), cc(B + 1, 0);
    for (int b = 0; b < B; ++b) {
      cu[b + 1] = cu[b] + L[b];
      cc[b + 1] = cc[b] + L[b] / r;
    }
    const int chunk = 1 + rng() % (T + 10);
    for (int t0 = 0; t0 < T; t0 += chunk) {
      const int nT = std::min(chunk, T - t0);
      const long long cap = item_cap(mode, B, chunk, mode == 2 ? 0 : n_cap, W, kb);
      std::vector<Item> items;
      std::vector<Record> recs;
      int parts = 0;
      for (int b = 0; b < B; ++b) {
        const SampleChunk sc = sample_chunk(cu[b], L[b], t0, nT);
        if (sc.pa >= sc.pb) continue;
        if (mode != 2) {
          const int rows = cmp_rows(sc, r, n_cap), nblk = cmp_blocks(sc, r, n_cap, kb);
          const int nch = n_chunks(sc);
          std::vector<int> clo(nblk), first(nblk);
          for (int k = 0; k < nblk; ++k) {
            clo[k] = cmp_clo(sc, r, k, kb);
            if (k > 0 && clo[k] < clo[k - 1]) fail("first query chunk of a block decreases");
            const int ni = nch - clo[k];
            if (ni < 1) fail("a visible block without items");
            first[k] = parts;
            recs.push_back({cc[b] + kb * k, std::min(kb, rows - kb * k), mode, parts, ni});
            parts += ni;
          }
          for (int c = 0; c < nch; ++c)
            for (int k = 0; k < nblk && clo[k] <= c; ++k) {
              const int qa = std::max(cmp_qlo(sc, r, k, kb), sc.pa + kCq * c);
              const int qb = std::min(sc.pb, sc.pa + kCq * (c + 1));
              items.push_back({cc[b] + kb * k, std::min(kb, rows - kb * k), mode, cu[b] + qa,
                               qb - qa, first[k] + (c - clo[k])});
            }
        }
        if (W > 0) {
          const int mlo = win_mlo(sc, W, kb), nm = win_mhi(sc, kb) - mlo;
          for (int i = 0; i < nm; ++i) {
            const int m = mlo + i;
            const WinBlock wb = win_block(sc, W, m, kb);
            if (wb.pieces > 0) recs.push_back({cu[b] + kb * m, wb.nk, 2, parts, wb.pieces});
            for (int e = 0; e < wb.pieces; ++e) {
              const int qa = wb.qlo + kCq * e;
              items.push_back({cu[b] + kb * m, wb.nk, 2, cu[b] + qa, std::min(kCq, wb.qhi - qa),
                               parts + e});
            }
            parts += wb.pieces;
          }
        }
      }
      if ((long long)items.size() > cap || (long long)recs.size() > cap || parts > cap)
        fail("items, partial slots or records beyond item_cap");
      // coverage: (query, compressed row j) and (query, raw row -1 - u)
      std::map<std::pair<int, int>, int> cover;
      for (const Item& it : items) {
        if (it.nq <= 0 || it.nq > kCq || it.nk <= 0 || it.nk > kb) fail("item out of shape");
        if (it.q0 < t0 || it.q0 + it.nq > t0 + nT) fail("item outside its query chunk");
        for (int t = it.q0; t < it.q0 + it.nq; ++t) {
          const int b = int(std::upper_bound(cu.begin(), cu.end(), t) - cu.begin()) - 1;
          const int p = t - cu[b];
          for (int x = 0; x < it.nk; ++x) {
            if (it.kind == 2) {
              const int u = it.key0 + x;
              if (u < cu[b] || u >= cu[b + 1]) fail("window row outside the query's sample");
              const int w0 = t - std::min(W, p + 1) + 1;
              if (u >= w0 && u <= t) cover[{t, -1 - u}]++;
            } else {
              const int jl = it.key0 + x - cc[b];
              if (jl < 0) fail("compressed row before the query's sample");
              if (jl < std::min((p + 1) / r, n_cap)) cover[{t, it.key0 + x}]++;
            }
          }
        }
      }
      for (int t = t0; t < t0 + nT; ++t) {
        const int b = int(std::upper_bound(cu.begin(), cu.end(), t) - cu.begin()) - 1;
        const int p = t - cu[b];
        if (mode != 2)
          for (int jl = 0; jl < std::min((p + 1) / r, n_cap); ++jl) {
            ++*pairs;
            if (cover[{t, cc[b] + jl}] != 1) fail("compressed pair not covered exactly once");
          }
        for (int u = t - std::min(W, p + 1) + 1; u <= t; ++u) {
          ++*pairs;
          if (cover[{t, -1 - u}] != 1) fail("window pair not covered exactly once");
        }
      }
      // partial slots: one per item; each record's slots are its block's items
      std::vector<int> owner(parts, -1);
      for (size_t i = 0; i < items.size(); ++i) {
        const int q = items[i].part;
        if (q < 0 || q >= parts || owner[q] >= 0) fail("partial slot missing or shared");
        else owner[q] = int(i);
      }
      for (const Record& rc : recs)
        for (int q = rc.first; q < rc.first + rc.count; ++q) {
          const int i = q < parts ? owner[q] : -1;
          if (i < 0 || items[i].key0 != rc.key0 || items[i].nk != rc.nk ||
              (items[i].kind == 2) != (rc.kind == 2))
            fail("record slot not an item of its block");
        }
    }
  }
  return fails;
}

}  // namespace

int main(int argc, char** argv) {
  const int trials = argc > 1 ? std::atoi(argv[1]) : 30;
  long long pairs = 0;
  int fails = 0;
  for (int kb : {128, 256}) fails += run(kb, trials, 1u + kb, &pairs);
  std::printf("pairs %lld failures %d\n", pairs, fails);
  return fails ? 1 : 0;
}
