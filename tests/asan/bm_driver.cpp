// Host-only driver of libpa's block manager and of the C ABI's argument validation, for
// a build with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_asan_host.py
// compiles it with g++ together with block_manager.cpp, api.cpp and launcher stubs).
//
// Reads one command per line on stdin and answers one line on stdout:
//   create N BS PC          -> ok | err S
//   add SID N t1 .. tN      -> ok CACHED | err S
//   append SID TOK          -> ok SLOT SRC DST | err S
//   fork PARENT CHILD       -> ok | err S
//   free SID                -> ok | err S
//   free_count              -> ok N
//   ctx SID                 -> ok L
//   tables W K s1 .. sK     -> ok bt[0..K*W) cl[0..K) | err S
//   slots SID FIRST COUNT   -> ok s[0..COUNT) | err S
//   ref B                   -> ok R
//   abi                     -> ok | bad I (the I-th validation case returned another status)
//   quit                    (destroys the manager and exits 0)
// Sanitizer reports go to stderr and end the process with a non-zero status.
#include <cstdint>
#include <cstdio>
#include <iostream>
#include <sstream>
#include <string>
#include <vector>

#include "../../include/pa.h"

namespace {

// Validation cases of the kernel entry points: every one is rejected (or is an empty
// call) on the host before any launch. Host addresses below are never dereferenced.
int abi_cases() {
  pa_kv_pool_t p = {(void*)0x1000, (void*)0x2000, nullptr, nullptr, 64, 16, 2, 128, PA_BF16};
  pa_kv_pool_t bad_bs = p;
  bad_bs.block_size = 8;
  pa_kv_pool_t fp8_noscale = p;
  fp8_noscale.dtype = PA_FP8_E4M3;
  pa_kv_pool_t bad_d = p;
  bad_d.head_dim = 96;
  void* const A = (void*)0x8000;
  const int64_t* sm = (const int64_t*)0x7000;
  const int32_t* bt = (const int32_t*)0xA000;
  const int32_t* cl = (const int32_t*)0xB000;
  const int32_t* cu = (const int32_t*)0xC000;
  struct Case { int got, want; };
  const Case cases[] = {
      {pa_store_kv(nullptr, A, A, PA_BF16, 4, 256, 128, 256, 128, sm, nullptr), PA_ERR_INVALID_ARG},
      {pa_store_kv(&p, A, A, PA_BF16, 0, 256, 128, 256, 128, sm, nullptr), PA_OK},
      {pa_store_kv(&p, A, A, PA_BF16, -1, 256, 128, 256, 128, sm, nullptr), PA_ERR_INVALID_ARG},
      {pa_store_kv(&p, A, A, PA_F32, 4, 256, 128, 256, 128, sm, nullptr), PA_ERR_INVALID_ARG},
      {pa_store_kv(&bad_bs, A, A, PA_BF16, 4, 256, 128, 256, 128, sm, nullptr), PA_ERR_UNSUPPORTED},
      {pa_store_kv(&fp8_noscale, A, A, PA_BF16, 4, 256, 128, 256, 128, sm, nullptr), PA_ERR_INVALID_ARG},
      {pa_store_kv(&bad_d, A, A, PA_BF16, 4, 256, 128, 256, 128, sm, nullptr), PA_ERR_UNSUPPORTED},
      {pa_store_kv(&p, A, A, PA_BF16, 4, -256, 128, 256, 128, sm, nullptr), PA_ERR_INVALID_ARG},
      {pa_decode(A, 1536, 128, A, 1536, 128, PA_BF16, 0, 12, &p, bt, 8, cl, 128, 0.1f, 0, nullptr, 0, nullptr), PA_OK},
      {pa_decode(A, 1536, 128, A, 1536, 128, PA_BF16, 2, 13, &p, bt, 8, cl, 128, 0.1f, 0, nullptr, 0, nullptr), PA_ERR_INVALID_ARG},
      {pa_decode(A, 1536, 128, A, 1536, 128, PA_BF16, 2, 18, &p, bt, 8, cl, 128, 0.1f, 0, nullptr, 0, nullptr), PA_ERR_UNSUPPORTED},
      {pa_decode(A, 1536, 128, A, 1536, 128, PA_BF16, 2, 12, &p, bt, 8, cl, 129, 0.1f, 0, nullptr, 0, nullptr), PA_ERR_INVALID_ARG},
      {pa_decode(A, 1536, 128, A, 1536, 128, PA_BF16, 2, 12, &p, bt, 8, cl, 128, -1.0f, 0, nullptr, 0, nullptr), PA_ERR_INVALID_ARG},
      {pa_decode(A, 1536, 128, A, 1536, 128, PA_BF16, 2, 12, &p, bt, 8, cl, 128, 0.1f, 16, nullptr, 0, nullptr), PA_ERR_WORKSPACE},
      {pa_decode(A, 1536, 128, A, 1536, 128, PA_BF16, 2, 12, &p, bt, 8, cl, 128, 0.1f, 8, nullptr, 0, nullptr), PA_ERR_INVALID_ARG},
      {pa_decode_step(A, 1536, 128, A, 1536, 128, PA_BF16, 2, 12, &p, A, A, PA_F32, 256, 128, 256, 128, sm, bt, 8, cl, 128, 0.1f, 128, nullptr, 0, nullptr), PA_ERR_INVALID_ARG},
      {pa_decode_step(A, 1536, 128, A, 1536, 128, PA_BF16, 2, 12, &p, nullptr, A, PA_BF16, 256, 128, 256, 128, sm, bt, 8, cl, 128, 0.1f, 128, nullptr, 0, nullptr), PA_ERR_INVALID_ARG},
      {pa_varlen_prefill(A, 1536, 128, A, 1536, 128, PA_BF16, cu, 2, 10, 5, 12, &p, bt, 8, cl, 128, 0.1f, 0, nullptr, 0, nullptr), PA_ERR_WORKSPACE},
      {pa_varlen_prefill(A, 1536, 128, A, 1536, 128, PA_BF16, cu, 2, 10, 200, 12, &p, bt, 8, cl, 128, 0.1f, 0, A, 1 << 20, nullptr), PA_ERR_INVALID_ARG},
      {pa_varlen_prefill(A, 1536, 128, A, 1536, 128, PA_BF16, cu, 2, 10, 5, 12, &p, bt, 8, cl, 128, 0.1f, 32, A, 1 << 20, nullptr), PA_ERR_INVALID_ARG},
      {pa_varlen_prefill(A, 1536, 128, A, 1536, 128, PA_BF16, cu, 0, 0, 5, 12, &p, bt, 8, cl, 128, 0.1f, 0, nullptr, 0, nullptr), PA_OK},
      {pa_rope_store_kv(&p, A, 1536, 128, 12, A, 1536, 128, A, A, PA_BF16, 4, 256, 128, 256, 128, sm, (const float*)A, (const float*)A, 0, sm, nullptr), PA_ERR_INVALID_ARG},
      {pa_copy_blocks(&p, bt, cl, 0, nullptr), PA_OK},
      {pa_copy_blocks(&p, nullptr, cl, 3, nullptr), PA_ERR_INVALID_ARG},
      {(int)pa_decode_workspace_bytes(2, 12, 2, 128, 128, 16) == 4096 + 2 * 12 * 8 * 129 * 4 ? PA_OK : -99, PA_OK},
      {(int)pa_decode_workspace_bytes(-2, 12, 2, 128, 128, 16), 0},
      {pa_decode_default_split_tokens(256, 8, 32768), 1024},
  };
  int i = 0;
  for (const Case& c : cases) {
    if (c.got != c.want) return i + 1;
    ++i;
  }
  return 0;
}

}  // namespace

int main() {
  pa_block_manager_t* bm = nullptr;
  std::string line;
  while (std::getline(std::cin, line)) {
    std::istringstream in(line);
    std::string cmd;
    in >> cmd;
    std::ostringstream out;
    if (cmd == "create") {
      long long n;
      int bs, pc;
      in >> n >> bs >> pc;
      if (bm) pa_bm_destroy(bm);
      bm = pa_bm_create(n, bs, pc);
      out << (bm ? "ok" : "err -1");
    } else if (cmd == "add") {
      long long sid, n;
      in >> sid >> n;
      std::vector<int32_t> t((size_t)n);
      for (auto& x : t) in >> x;
      int64_t cached = -1;
      const int st = pa_bm_add_sequence(bm, sid, t.data(), n, &cached);
      if (st == PA_OK) out << "ok " << cached; else out << "err " << st;
    } else if (cmd == "append") {
      long long sid;
      int tok;
      in >> sid >> tok;
      int64_t slot = -7;
      int32_t src = -7, dst = -7;
      const int st = pa_bm_append_token(bm, sid, tok, &slot, &src, &dst);
      if (st == PA_OK) out << "ok " << slot << " " << src << " " << dst; else out << "err " << st;
    } else if (cmd == "fork") {
      long long a, b;
      in >> a >> b;
      const int st = pa_bm_fork(bm, a, b);
      if (st == PA_OK) out << "ok"; else out << "err " << st;
    } else if (cmd == "free") {
      long long sid;
      in >> sid;
      const int st = pa_bm_free_sequence(bm, sid);
      if (st == PA_OK) out << "ok"; else out << "err " << st;
    } else if (cmd == "free_count") {
      out << "ok " << pa_bm_num_free_blocks(bm);
    } else if (cmd == "ctx") {
      long long sid;
      in >> sid;
      out << "ok " << pa_bm_context_len(bm, sid);
    } else if (cmd == "tables") {
      int w, k;
      in >> w >> k;
      std::vector<int64_t> ids((size_t)k);
      for (auto& x : ids) in >> x;
      std::vector<int32_t> tab((size_t)k * w), cl((size_t)k);
      const int st = pa_bm_block_tables(bm, ids.data(), k, w, tab.data(), cl.data());
      if (st == PA_OK) {
        out << "ok";
        for (int32_t x : tab) out << " " << x;
        for (int32_t x : cl) out << " " << x;
      } else {
        out << "err " << st;
      }
    } else if (cmd == "slots") {
      long long sid, first, count;
      in >> sid >> first >> count;
      std::vector<int64_t> s((size_t)(count > 0 ? count : 0));
      const int st = pa_bm_slots(bm, sid, first, count, s.data());
      if (st == PA_OK) {
        out << "ok";
        for (int64_t x : s) out << " " << x;
      } else {
        out << "err " << st;
      }
    } else if (cmd == "ref") {
      int b;
      in >> b;
      out << "ok " << pa_bm_block_refcount(bm, b);
    } else if (cmd == "abi") {
      const int bad = abi_cases();
      if (bad == 0) out << "ok"; else out << "bad " << bad;
    } else if (cmd == "quit") {
      break;
    } else {
      out << "err unknown";
    }
    std::cout << out.str() << std::endl;
  }
  if (bm) pa_bm_destroy(bm);
  return 0;
}
