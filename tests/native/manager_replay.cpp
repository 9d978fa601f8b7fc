// Replays a text trace of block-manager operations through the C ABI of
// libpkv's host manager and checks its invariants after every operation.
// Built by tests/test_manager_sanitizers.py with AddressSanitizer and
// UndefinedBehaviorSanitizer around manager.cpp (host code only).
//
// First line: num_blocks block_size sort_on_release.  Then one op per line:
//   P id n          allocate_for_prefill          A id        append one
//   B k id...       batched append                F id        free
//   C n             can_allocate                  S d id n    share prefix
//   T id n          append_tokens                 O id / I id swap out / in
//   M e k (id n)... admit_batch (e = extend_live) Q           drain copies
// Exit status 0 when every op ran and the invariants held after each, 2 on
// a violated invariant, 3 on a malformed trace.
#include <cstdio>
#include <cstdlib>
#include <vector>

#include "pkv.h"

int main() {
  int n_blocks = 0, bs = 0, sort = 0;
  if (std::scanf("%d %d %d", &n_blocks, &bs, &sort) != 3) return 3;
  pkv_manager* m = pkv_manager_create(n_blocks, bs, nullptr, sort ? PKV_SORT_ON_RELEASE : 0u);
  if (!m) return 3;
  std::vector<int64_t> slots(1 << 16);
  std::vector<int32_t> ids32(n_blocks), a(n_blocks), b(n_blocks), lens(4096);
  std::vector<int64_t> ids64(4096);
  std::vector<int32_t> chunk(4096);
  char op[4];
  long ops = 0, ok = 0;
  while (std::scanf("%3s", op) == 1) {
    int st = 0;
    long long id = 0, id2 = 0;
    int n = 0, k = 0, e = 0, cnt = 0;
    switch (op[0]) {
      case 'P':
        if (std::scanf("%lld %d", &id, &n) != 2) return 3;
        st = pkv_allocate_for_prefill(m, id, n, n >= 0 && n <= (1 << 16) ? slots.data() : nullptr);
        break;
      case 'A':
        if (std::scanf("%lld", &id) != 1) return 3;
        st = pkv_append_slot_for_decode(m, id, slots.data());
        break;
      case 'B':
        if (std::scanf("%d", &k) != 1 || k < 0 || k > 4096) return 3;
        for (int i = 0; i < k; ++i)
          if (std::scanf("%lld", &id) != 1) return 3; else ids64[i] = id;
        st = pkv_append_slots_for_decode(m, ids64.data(), k, slots.data(), lens.data(), chunk.data());
        break;
      case 'F':
        if (std::scanf("%lld", &id) != 1) return 3;
        st = pkv_free_sequence(m, id);
        break;
      case 'C':
        if (std::scanf("%d", &n) != 1) return 3;
        st = pkv_can_allocate(m, n);
        break;
      case 'S':
        if (std::scanf("%lld %lld %d", &id, &id2, &n) != 3) return 3;
        st = pkv_share_prefix(m, id, id2, n);
        break;
      case 'T':
        if (std::scanf("%lld %d", &id, &n) != 2) return 3;
        st = pkv_append_tokens(m, id, n, n >= 0 && n <= (1 << 16) ? slots.data() : nullptr);
        break;
      case 'O':
        if (std::scanf("%lld", &id) != 1) return 3;
        st = pkv_swap_out(m, id, ids32.data(), n_blocks, &cnt);
        break;
      case 'I':
        if (std::scanf("%lld", &id) != 1) return 3;
        st = pkv_swap_in(m, id, ids32.data(), n_blocks, &cnt);
        break;
      case 'M': {
        if (std::scanf("%d %d", &e, &k) != 2 || k < 0 || k > 4096) return 3;
        long long total = 0;
        for (int i = 0; i < k; ++i) {
          if (std::scanf("%lld %d", &id, &n) != 2) return 3;
          ids64[i] = id;
          chunk[i] = n;
          if (n > 0) total += n;
        }
        st = pkv_admit_batch(m, ids64.data(), chunk.data(), k, e, total <= (1 << 16) ? slots.data() : nullptr,
                             lens.data());
        break;
      }
      case 'Q':
        st = pkv_take_block_copies(m, a.data(), b.data(), n_blocks, &cnt);
        break;
      default:
        return 3;
    }
    ++ops;
    if (st >= 0) ++ok;
    if (pkv_check_invariants(m) != PKV_OK) {
      std::fprintf(stderr, "invariant violated after op %ld (%s)\n", ops, op);
      return 2;
    }
  }
  std::printf("%ld ops, %ld succeeded, %d free blocks\n", ops, ok, pkv_num_free_blocks(m));
  pkv_manager_destroy(m);
  return 0;
}
