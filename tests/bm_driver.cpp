// Command-line driver of the host block manager (pkv_bm_* in pagedkv.h), for
// tests that build it together with block_manager.cpp under the address and
// undefined-behaviour sanitizers.  It reads one command per line on stdin and
// answers each with one line on stdout, so a test can feed the same calls to
// the oracle's block manager and compare the two transcripts.
//
//   create NB BS o_0 .. o_{NB-1}      -> ok
//   add SEQ N                         -> ok slot_0 .. slot_{N-1}   | err CODE
//   addc SEQ N id_0 .. id_{N-1}       -> ok CACHED slot_0 ..       | err CODE
//   fork PARENT CHILD                 -> ok                        | err CODE
//   app SEQ                           -> ok SLOT SRC DST           | err CODE
//   tok SEQ ID                        -> ok SLOT SRC DST           | err CODE
//   step N s_0 .. s_{N-1}             -> ok slots.. ; src dst ..   | err CODE
//   free SEQ                          -> ok                        | err CODE
//   state N s_0 .. s_{N-1}            -> free F evict E list .. ; ref .. ; then per
//                                        sequence: LEN WASTE NBLK table ..
//
// Test code only: it is not part of the library.

#include <cstdint>
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "pagedkv.h"

namespace {

void put_err(pkv_status st) { std::printf("err %d\n", static_cast<int>(st)); }

}  // namespace

int main() {
  std::ios::sync_with_stdio(false);
  pkv_block_manager* bm = nullptr;
  int32_t nb = 0;
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string cmd;
    if (!(in >> cmd)) continue;
    if (cmd == "create") {
      int32_t bs = 0;
      in >> nb >> bs;
      std::vector<int32_t> order(static_cast<size_t>(nb));
      for (auto& o : order) in >> o;
      if (bm) pkv_bm_destroy(bm);
      bm = pkv_bm_create(nb, bs, order.data());
      std::printf(bm ? "ok\n" : "err 1\n");
    } else if (!bm) {
      std::printf("err 1\n");
    } else if (cmd == "add" || cmd == "addc") {
      int32_t seq = 0, n = 0;
      in >> seq >> n;
      std::vector<int32_t> ids(static_cast<size_t>(n > 0 ? n : 1));
      if (cmd == "addc")
        for (int32_t i = 0; i < n; ++i) in >> ids[i];
      // exactly n slots: a write past them is what the sanitizer is here to catch
      std::vector<int32_t> slots(static_cast<size_t>(n));
      int32_t cached = 0;
      pkv_status st = cmd == "add" ? pkv_bm_add(bm, seq, n, n ? slots.data() : nullptr)
                                   : pkv_bm_add_cached(bm, seq, n, ids.data(), n ? slots.data() : nullptr, &cached);
      if (st != PKV_OK) {
        put_err(st);
        continue;
      }
      std::printf("ok");
      if (cmd == "addc") std::printf(" %d", cached);
      for (int32_t s : slots) std::printf(" %d", s);
      std::printf("\n");
    } else if (cmd == "fork") {
      int32_t p = 0, c = 0;
      in >> p >> c;
      pkv_status st = pkv_bm_fork(bm, p, c);
      if (st != PKV_OK) put_err(st);
      else std::printf("ok\n");
    } else if (cmd == "app" || cmd == "tok") {
      int32_t seq = 0, id = 0, slot = -1, pair[2] = {-1, -1};
      in >> seq;
      if (cmd == "tok") in >> id;
      pkv_status st = cmd == "app" ? pkv_bm_append_slot(bm, seq, &slot, pair)
                                   : pkv_bm_append_token(bm, seq, id, &slot, pair);
      if (st != PKV_OK) put_err(st);
      else std::printf("ok %d %d %d\n", slot, pair[0], pair[1]);
    } else if (cmd == "step") {
      int32_t n = 0;
      in >> n;
      std::vector<int32_t> seqs(static_cast<size_t>(n));
      for (auto& s : seqs) in >> s;
      std::vector<int32_t> slots(static_cast<size_t>(n)), pairs(static_cast<size_t>(2 * n));
      int32_t np = 0;
      pkv_status st = pkv_bm_step(bm, seqs.data(), n, slots.data(), pairs.data(), &np);
      if (st != PKV_OK) {
        put_err(st);
        continue;
      }
      std::printf("ok");
      for (int32_t s : slots) std::printf(" %d", s);
      std::printf(" ;");
      for (int32_t i = 0; i < 2 * np; ++i) std::printf(" %d", pairs[i]);
      std::printf("\n");
    } else if (cmd == "free") {
      int32_t seq = 0;
      in >> seq;
      pkv_status st = pkv_bm_free(bm, seq);
      if (st != PKV_OK) put_err(st);
      else std::printf("ok\n");
    } else if (cmd == "state") {
      int32_t n = 0;
      in >> n;
      std::vector<int32_t> seqs(static_cast<size_t>(n));
      for (auto& s : seqs) in >> s;
      int32_t nfree_list = pkv_bm_free_list(bm, nullptr, 0);
      std::vector<int32_t> fl(static_cast<size_t>(nfree_list));
      pkv_bm_free_list(bm, fl.data(), nfree_list);
      std::printf("free %d evict %d list", pkv_bm_num_free(bm), pkv_bm_num_evictable(bm));
      for (int32_t b : fl) std::printf(" %d", b);
      std::printf(" ; ref");
      for (int32_t b = 0; b < nb; ++b) std::printf(" %d", pkv_bm_refcount(bm, b));
      for (int32_t s : seqs) {
        int32_t nblk = pkv_bm_num_seq_blocks(bm, s);
        int32_t mb = nblk > 0 ? nblk : 1;
        std::vector<int32_t> table(static_cast<size_t>(mb));
        int32_t len = -1;
        pkv_status st = pkv_bm_block_table(bm, &s, 1, mb, table.data(), &len);
        std::printf(" ; %d %d %d", pkv_bm_length(bm, s), pkv_bm_waste(bm, s), nblk);
        if (st != PKV_OK) {
          std::printf(" err %d", static_cast<int>(st));
          continue;
        }
        for (int32_t i = 0; i < nblk; ++i) std::printf(" %d", table[i]);
      }
      std::printf("\n");
    } else {
      std::printf("err 1\n");
    }
    std::fflush(stdout);
  }
  if (bm) pkv_bm_destroy(bm);
  return 0;
}
