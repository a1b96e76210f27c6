// Status codes, the thread-local last error, and the host-only batch validator.
#include <cmath>
#include <cstdio>
#include <string>
#include <unordered_map>
#include <vector>

#include "cb_internal.h"

namespace cb {

static thread_local std::string g_last_error;

int fail(int status, const std::string& msg) {
  g_last_error = msg;
  return status;
}

int ok() {
  g_last_error.clear();
  return CB_OK;
}

}  // namespace cb

extern "C" const char* cb_status_string(int status) {
  switch (status) {
    case CB_OK: return "CB_OK";
    case CB_ERR_INVALID_ARG: return "CB_ERR_INVALID_ARG";
    case CB_ERR_UNSUPPORTED: return "CB_ERR_UNSUPPORTED";
    case CB_ERR_WORKSPACE: return "CB_ERR_WORKSPACE";
    case CB_ERR_HIP: return "CB_ERR_HIP";
    case CB_ERR_OUT_OF_BLOCKS: return "CB_ERR_OUT_OF_BLOCKS";
    default: return "CB_ERR_UNKNOWN";
  }
}

extern "C" const char* cb_last_error(void) { return cb::g_last_error.c_str(); }

namespace {

std::string fmt(const char* f, long long a = 0, long long b = 0, long long c = 0,
                long long d = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, f, a, b, c, d);
  return buf;
}

}  // namespace

extern "C" int cb_validate_batch(const int32_t* cu, const int32_t* kv_lens,
                                 const int32_t* block_tables, const int32_t* slot_mapping,
                                 int32_t num_seqs, int32_t num_tokens, int32_t max_blocks_per_seq,
                                 int32_t block_size, int64_t num_blocks, int32_t max_q_len,
                                 int32_t max_kv_len) {
  using cb::fail;
  const int E = CB_ERR_INVALID_ARG;
  if (block_size < 4) return fail(E, fmt("block_size must be at least 4, got %lld", block_size));
  if (num_seqs < 0 || num_tokens < 0) return fail(E, "negative num_seqs or num_tokens");
  if (num_blocks < 1) return fail(E, "num_blocks must be positive");
  if (num_blocks * (int64_t)block_size > INT32_MAX)
    return fail(E, "num_blocks * block_size must stay below 2^31 (int32 slots)");
  if (!cu) return fail(E, "cu_seqlens_q is NULL");
  if (num_seqs > 0 && (!kv_lens || !block_tables)) return fail(E, "kv_lens or block_tables NULL");
  if (num_seqs > 0 && max_blocks_per_seq < 1) return fail(E, "max_blocks_per_seq must be >= 1");
  if (cu[0] != 0) return fail(E, fmt("cu_seqlens_q[0] = %lld, must be 0", cu[0]));
  if (cu[num_seqs] != num_tokens)
    return fail(E, fmt("cu_seqlens_q[S] = %lld but num_tokens = %lld", cu[num_seqs], num_tokens));

  std::vector<int32_t> refs(static_cast<size_t>(num_blocks), 0);
  for (int32_t s = 0; s < num_seqs; ++s) {
    const int64_t q = (int64_t)cu[s + 1] - cu[s];
    const int64_t L = kv_lens[s];
    if (q < 0) return fail(E, fmt("cu_seqlens_q decreases at sequence %lld", s));
    if (q == 0) return fail(E, fmt("sequence %lld has no tokens in this step (zero-length row)", s));
    if (L < q) return fail(E, fmt("sequence %lld: kv_len %lld < q_len %lld", s, L, q));
    if (q > max_q_len) return fail(E, fmt("sequence %lld: q_len %lld > max_q_len %lld", s, q, max_q_len));
    if (L > max_kv_len)
      return fail(E, fmt("sequence %lld: kv_len %lld > max_kv_len %lld", s, L, max_kv_len));
    if (L > (int64_t)max_blocks_per_seq * block_size)
      return fail(E, fmt("sequence %lld: kv_len %lld exceeds its table capacity %lld", s, L,
                         (int64_t)max_blocks_per_seq * block_size));
    const int64_t nb = cb::ceil_div(L, block_size);
    const int32_t* row = block_tables + (int64_t)s * max_blocks_per_seq;
    for (int64_t j = 0; j < nb; ++j) {
      if (row[j] < 0 || row[j] >= num_blocks)
        return fail(E, fmt("sequence %lld: table entry %lld = %lld out of [0, num_blocks)", s, j,
                           row[j]));
      refs[row[j]] += 1;
    }
  }
  if (slot_mapping) {
    const int64_t nslots = num_blocks * (int64_t)block_size;
    std::unordered_map<int32_t, int32_t> seen;
    seen.reserve(static_cast<size_t>(num_tokens) * 2);
    for (int32_t t = 0; t < num_tokens; ++t) {
      const int32_t sl = slot_mapping[t];
      if (sl == -1) continue;
      if (sl < 0 || sl >= nslots)
        return fail(E, fmt("token %lld: slot %lld out of range", t, sl));
      auto it = seen.find(sl);
      if (it != seen.end())
        return fail(E, fmt("tokens %lld and %lld write the same slot %lld", it->second, t, sl));
      seen.emplace(sl, t);
      if (refs[sl / block_size] > 1)
        return fail(E, fmt("token %lld writes slot %lld inside block %lld, which more than one "
                           "table entry references (copy the block first)",
                           t, sl, sl / block_size));
    }
  }
  return cb::ok();
}
