// C-ABI entry points of the paged KV-cache library: argument checks, the
// partition plan of split-context decode, and kernel launches on the caller's
// stream.  Nothing here allocates, frees, synchronises or reads device memory.
#include <algorithm>
#include <climits>
#include <cstdint>
#include <numeric>
#include <vector>

#include "kernels.h"
#include "pkv.h"

namespace {

constexpr double kLog2e = 1.4426950408889634;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t align256(size_t n) { return (n + 255) & ~static_cast<size_t>(255); }

bool dtype_ok(int32_t dtype) { return dtype == PKV_BF16 || dtype == PKV_FP16; }

bool block_size_ok(int32_t bs) { return bs >= 16 && bs <= 1024 && bs % 16 == 0; }

// Compute units the automatic plan is sized for (MI355X).
constexpr int64_t kPlanCUs = 256;
// XCDs the launch's work-item ranges are spread over (MI355X), as in xcd_remap.
constexpr int kXcds = 8;

// Tokens per partition for the automatic plan, 0 for one pass without merge.
// One workgroup per (sequence, kv head) reads a whole context when there are
// at least two such units per compute unit and no context is longer than
// 4096 tokens: on the ragged Llama-3.2-1B batch this is faster than any split
// plus the merge pass.  Otherwise contexts are cut into partitions of
// 1536 tokens, halved (down to 192) until there are at least two (sequence,
// kv head, partition) workgroups per compute unit.  1536 tokens (24 sub-tiles
// per wave of a four-wave workgroup) measured faster than 1024, 2048 and 4096
// on the long-context batch (16 sequences of 4096-8192 tokens: 38.9 us vs
// 40.0, 41.0, 39.4) and on the 16-layer continuous-batching step.
int32_t auto_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t max_ctx) {
  const int64_t units = static_cast<int64_t>(num_seqs) * num_kv_heads;
  if (units >= 2 * kPlanCUs && max_ctx <= 4096) return 0;
  int32_t pt = 1536;
  while (pt > 256 && units * ((max_ctx + pt - 1) / pt) < 2 * kPlanCUs) pt /= 2;
  return pt >= max_ctx ? 0 : pt;
}

struct Plan {
  int32_t part_tokens;  // multiple of 16
  int32_t num_parts;
};

Plan make_plan(int32_t num_seqs, int32_t num_kv_heads, int32_t max_ctx, int32_t partition_tokens) {
  int32_t pt = partition_tokens > 0 ? partition_tokens : auto_partition(num_seqs, num_kv_heads, max_ctx);
  if (pt <= 0 || pt >= max_ctx) pt = max_ctx <= 16 ? 16 : ((max_ctx + 15) / 16) * 16;
  // a workgroup of the MFMA kernel takes at most kMaxPartitionTokens tokens
  if (pt > pkv::kMaxPartitionTokens) pt = pkv::kMaxPartitionTokens;
  const int32_t parts = max_ctx <= pt ? 1 : (max_ctx + pt - 1) / pt;
  return {pt, parts};
}

// Partial-state bytes: num_parts + prefix_chunks slots per (sequence, q head),
// none when a single pass writes every output.
size_t workspace_for(int32_t num_seqs, int32_t num_q_heads, int32_t head_dim, const Plan& plan,
                     int32_t prefix_chunks = 0) {
  const int64_t slots = static_cast<int64_t>(plan.num_parts) + prefix_chunks;
  if (slots <= 1) return 0;
  const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * slots;
  return align256(rows * head_dim * sizeof(float)) + 2 * align256(rows * sizeof(float));
}

// Tokens of a shared prefix one prefix unit (a wave) takes: half the longest
// prefix, between 64 and 1024 tokens (a wave holds the ids of at most 64
// sub-tiles).  On the 16-layer step (512-token prefixes) halves measured
// 42.4 us per layer, whole prefixes 44.4, quarters 43.6 and eighths 49.8.
int32_t prefix_chunk_tokens(int32_t max_prefix_len) {
  int32_t c = (max_prefix_len + 1) / 2;
  c = (c + 15) / 16 * 16;
  return c < 64 ? 64 : (c > 1024 ? 1024 : c);
}

int32_t prefix_chunk_count(int32_t max_prefix_len) {
  if (max_prefix_len <= 0) return 0;
  const int32_t c = prefix_chunk_tokens(max_prefix_len);
  return (max_prefix_len + c - 1) / c;
}

// Auto-plan workspace bound over every longest context up to max_context_len
// (the automatic plan is not monotone in it; plans change only at multiples of 16).
size_t auto_workspace(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t max_context_len, int32_t prefix_chunks);

// Deal n entries of the given weights (tokens) to the XCDs' contiguous ranges
// of a launch, heaviest first, each to the group with the least weight so far
// that has room (group x holds ceil(n/8) entries for x < n % 8, floor(n/8)
// otherwise, as xcd_remap splits the items); within a group the entries keep
// the heaviest-first order.  Returns the entry order.
std::vector<int32_t> deal_to_xcds(const std::vector<int64_t>& weight) {
  const int32_t n = static_cast<int32_t>(weight.size());
  std::vector<int32_t> by_w(n);
  std::iota(by_w.begin(), by_w.end(), 0);
  std::stable_sort(by_w.begin(), by_w.end(), [&](int32_t a, int32_t b) { return weight[a] > weight[b]; });
  std::vector<std::vector<int32_t>> groups(kXcds);
  std::vector<int64_t> load(kXcds, 0);
  const int32_t base = n / kXcds, extra = n % kXcds;
  for (const int32_t e : by_w) {
    int best = -1;
    for (int g = 0; g < kXcds; ++g) {
      const int32_t cap = base + (g < extra ? 1 : 0);
      if (static_cast<int32_t>(groups[g].size()) >= cap) continue;
      if (best < 0 || load[g] < load[best]) best = g;
    }
    groups[best].push_back(e);
    load[best] += weight[e] > 0 ? weight[e] : 0;
  }
  std::vector<int32_t> order;
  order.reserve(n);
  for (const auto& g : groups) order.insert(order.end(), g.begin(), g.end());
  return order;
}

// The automatic plan is not monotone in the longest context (a shorter one
// may be cut into more, smaller partitions), so report the most any longest
// context up to max_context_len needs: one workspace then serves every later
// call whose bound is at most this one.
size_t auto_workspace(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t max_context_len, int32_t prefix_chunks) {
  size_t need = 0;
  for (int32_t m = 16; m < max_context_len + 16; m += 16) {
    const Plan plan = make_plan(num_seqs, num_kv_heads, m < max_context_len ? m : max_context_len, 0);
    const size_t w = workspace_for(num_seqs, num_q_heads, head_dim, plan, prefix_chunks);
    if (w > need) need = w;
  }
  return need;
}

}  // namespace

extern "C" {

const char* pkv_status_str(int status) {
  switch (status) {
    case PKV_OK: return "ok";
    case PKV_E_NULL: return "required pointer is NULL";
    case PKV_E_SHAPE: return "sizes inconsistent, out of range or misaligned";
    case PKV_E_UNSUPPORTED: return "dtype, head_dim, block_size or GQA group not supported";
    case PKV_E_WORKSPACE: return "workspace missing or too small";
    case PKV_E_HIP: return "HIP kernel launch failed";
    case PKV_E_NOMEM: return "not enough free blocks";
    case PKV_E_NOSEQ: return "unknown sequence id";
    case PKV_E_EXISTS: return "sequence id already present";
    default: return "unknown status";
  }
}

int pkv_kv_append(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                  void* k_cache, void* v_cache, int32_t num_blocks, int32_t block_size,
                  int32_t num_kv_heads, int32_t head_dim, int32_t dtype, hipStream_t stream) {
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PKV_E_SHAPE;
  if (!dtype_ok(dtype) || !block_size_ok(block_size) || head_dim <= 0 || head_dim % 8 || head_dim > 512)
    return PKV_E_UNSUPPORTED;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PKV_E_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_E_SHAPE;
  if (static_cast<int64_t>(num_tokens) * num_kv_heads * (head_dim / 8) > static_cast<int64_t>(INT_MAX) * 256)
    return PKV_E_SHAPE;
  pkv::AppendParams p;
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.slot_mapping = slot_mapping;
  p.k_cache = static_cast<uint16_t*>(k_cache);
  p.v_cache = static_cast<uint16_t*>(v_cache);
  p.num_tokens = num_tokens;
  p.num_blocks = num_blocks;
  p.block_size = block_size;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  return pkv::launch_kv_append(p, stream) == hipSuccess ? PKV_OK : PKV_E_HIP;
}

int pkv_decode_supported(int32_t impl, int32_t dtype, int32_t head_dim, int32_t group) {
  if (!dtype_ok(dtype)) return 0;
  switch (impl) {
    case PKV_IMPL_AUTO:
      return pkv::simt_supported(dtype, head_dim, group) || pkv::mfma_supported(dtype, head_dim, group);
    case PKV_IMPL_SIMT: return pkv::simt_supported(dtype, head_dim, group);
    case PKV_IMPL_MFMA: return pkv::mfma_supported(dtype, head_dim, group);
    default: return 0;
  }
}

int32_t pkv_decode_plan_partition(int32_t num_seqs, int32_t num_kv_heads, int32_t block_size,
                                  int32_t max_context_len) {
  (void)block_size;
  if (num_seqs <= 0 || num_kv_heads <= 0 || max_context_len <= 0) return 0;
  const Plan plan = make_plan(num_seqs, num_kv_heads, max_context_len, 0);
  return plan.num_parts > 1 ? plan.part_tokens : 0;
}

int pkv_decode_schedule(const int32_t* context_lens, int32_t num_seqs, int32_t* seq_order) {
  if (num_seqs < 0) return PKV_E_SHAPE;
  if (num_seqs == 0) return PKV_OK;
  if (!context_lens || !seq_order) return PKV_E_NULL;
  // longest context first (ties: lower index first), dealt to the XCD groups
  std::vector<int64_t> w(num_seqs);
  for (int32_t i = 0; i < num_seqs; ++i) w[i] = context_lens[i];
  const std::vector<int32_t> order = deal_to_xcds(w);
  std::copy(order.begin(), order.end(), seq_order);
  return PKV_OK;
}

int pkv_decode_work_list(const int32_t* context_lens, const int32_t* prefix_len, int32_t num_seqs,
                         int32_t num_kv_heads, int32_t max_context_len, int32_t partition_tokens, int32_t* work,
                         int32_t max_work, int32_t* num_work) {
  if (num_seqs < 0 || num_kv_heads <= 0 || num_kv_heads > 0x7fff || max_context_len < 0 || max_work < 0)
    return PKV_E_SHAPE;
  if (partition_tokens < 0 || partition_tokens % 16) return PKV_E_SHAPE;
  if (!num_work) return PKV_E_NULL;
  *num_work = 0;
  if (num_seqs == 0) return PKV_OK;
  if (!context_lens || (max_work > 0 && !work)) return PKV_E_NULL;
  // the partition plan and workgroup size the decode call uses for the same sizes
  const Plan plan = make_plan(num_seqs, num_kv_heads, max_context_len, partition_tokens);
  if (plan.num_parts > 0xffff) return PKV_E_SHAPE;
  const int64_t pt = plan.part_tokens;
  const int32_t nw = pkv::decode_workgroup_waves(plan.num_parts, plan.part_tokens);
  // entries of sequence i: es[first[i] .. first[i+1]), one per workgroup
  std::vector<int32_t> first(num_seqs + 1, 0), es, ey;
  std::vector<int64_t> tokens(num_seqs, 0);
  for (int32_t i = 0; i < num_seqs; ++i) {
    const int64_t L = context_lens[i];
    int64_t pl = prefix_len ? prefix_len[i] : 0;
    // a length the kernel rejects is answered by partition 0 alone
    if (pl < 0 || pl % 16 || (pl > 0 && pl > L - 1)) pl = 0;
    const bool bad = L <= 0 || L > max_context_len;
    const int64_t n = bad ? 1 : std::min<int64_t>(std::max<int64_t>((L - pl + pt - 1) / pt, 1), plan.num_parts);
    for (int64_t k = 0; k < n; ++k) {
      const int64_t toks = bad ? 0 : std::min<int64_t>(pt, L - pl - k * pt);
      tokens[i] += toks;
      if (toks <= pkv::kWaveModeMaxTokens) {
        // wave mode: one workgroup per nw kv heads
        for (int32_t h = 0; h < num_kv_heads; h += nw) {
          es.push_back(i);
          ey.push_back(static_cast<int32_t>(static_cast<uint32_t>(k) | (static_cast<uint32_t>(h) << 16) | (1u << 31)));
        }
      } else {
        for (int32_t h = 0; h < num_kv_heads; ++h) {
          es.push_back(i);
          ey.push_back(static_cast<int32_t>(static_cast<uint32_t>(k) | (static_cast<uint32_t>(h) << 16)));
        }
      }
    }
    first[i + 1] = static_cast<int32_t>(es.size());
  }
  // Whole sequences dealt to the 8 XCD groups by tokens (longest first, to the
  // group with the fewest tokens so far, then the fewest entries), each
  // group's entries padded with skipped entries (sequence -1) to the largest
  // group's count, so that xcd_remap's equal ranges are the groups.  Keeping a
  // sequence's partitions on one XCD measured faster than dealing partitions
  // one by one (long contexts in 1536-token partitions: 39.9 us against 46.1
  // per launch).
  std::vector<int32_t> by(num_seqs);
  std::iota(by.begin(), by.end(), 0);
  std::stable_sort(by.begin(), by.end(), [&](int32_t a, int32_t b) { return tokens[a] > tokens[b]; });
  std::vector<std::vector<int32_t>> g(kXcds);
  std::vector<int64_t> load(kXcds, 0);
  for (const int32_t sq : by) {
    int best = 0;
    for (int x = 1; x < kXcds; ++x)
      if (load[x] < load[best] || (load[x] == load[best] && g[x].size() < g[best].size())) best = x;
    for (int32_t e = first[sq]; e < first[sq + 1]; ++e) g[best].push_back(e);
    load[best] += tokens[sq];
  }
  size_t mx = 0;
  for (const auto& v : g) mx = std::max(mx, v.size());
  if (static_cast<int64_t>(mx) * kXcds > INT_MAX) return PKV_E_SHAPE;
  if (static_cast<int64_t>(mx) * kXcds > max_work) {
    *num_work = static_cast<int32_t>(mx * kXcds);  // the size needed
    return PKV_E_SHAPE;
  }
  size_t k = 0;
  for (const auto& v : g)
    for (size_t j = 0; j < mx; ++j) {
      work[2 * k] = j < v.size() ? es[v[j]] : -1;
      work[2 * k + 1] = j < v.size() ? ey[v[j]] : 0;
      ++k;
    }
  *num_work = static_cast<int32_t>(k);
  return PKV_OK;
}

size_t pkv_decode_workspace_bytes_ex(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                     int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                     int32_t partition_tokens) {
  return pkv_decode_prefix_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                           max_context_len, 0, partition_tokens);
}

size_t pkv_decode_prefix_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                         int32_t head_dim, int32_t block_size, int32_t max_context_len,
                                         int32_t max_prefix_len, int32_t partition_tokens) {
  (void)block_size;
  if (num_seqs <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0 || max_context_len <= 0)
    return 0;
  const int32_t chunks = prefix_chunk_count(max_prefix_len);
  if (partition_tokens > 0) {
    const Plan plan = make_plan(num_seqs, num_kv_heads, max_context_len, partition_tokens);
    return workspace_for(num_seqs, num_q_heads, head_dim, plan, chunks);
  }
  return auto_workspace(num_seqs, num_q_heads, num_kv_heads, head_dim, max_context_len, chunks);
}

size_t pkv_decode_workspace_bytes(int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                  int32_t head_dim, int32_t block_size, int32_t max_context_len) {
  return pkv_decode_workspace_bytes_ex(num_seqs, num_q_heads, num_kv_heads, head_dim, block_size,
                                       max_context_len, 0);
}

namespace {

// Shared body of the decode entry points; `app` carries the fused append
// (k_new, v_new, slot_mapping) or nulls.
struct FusedAppend {
  const void* k_new;
  const void* v_new;
  const int64_t* slot_mapping;
};

// Scales of FP8 (E4M3) pools (nullptr: 16-bit pools).
struct Fp8Scales {
  float k, v;
};

// Shared-prefix work (nullptr: none); device arrays as pkv_paged_attn_decode_prefix takes them.
struct PrefixDesc {
  const int32_t* prefix_len;
  const int32_t* prefix_items;
  int32_t num_items, max_prefix_len;
};

bool scale_ok(float s) { return s > 0.f && s <= 3.4e38f; }  // positive and finite (NaN fails both)

int decode_call(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len, float scale,
                void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                int32_t block_size, int32_t num_blocks, int32_t dtype, void* workspace, size_t workspace_bytes,
                int32_t partition_tokens, int32_t impl, const FusedAppend& app, const Fp8Scales* fp8,
                const int32_t* seq_order, hipStream_t stream, const PrefixDesc* pre = nullptr,
                const int32_t* work = nullptr, int32_t num_work = 0) {
  if (num_seqs < 0 || num_q_heads <= 0 || num_kv_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0 ||
      max_context_len < 0)
    return PKV_E_SHAPE;
  if (num_q_heads % num_kv_heads) return PKV_E_SHAPE;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return PKV_E_SHAPE;
  if (partition_tokens < 0 || partition_tokens % 16) return PKV_E_SHAPE;
  if (!dtype_ok(dtype) || !block_size_ok(block_size)) return PKV_E_UNSUPPORTED;
  // sub-tile indices of the pool are 32-bit inside the kernels
  if (static_cast<int64_t>(num_blocks) * num_kv_heads * (block_size / 16) > INT_MAX) return PKV_E_SHAPE;
  const int32_t group = num_q_heads / num_kv_heads;
  const bool simt_ok = pkv::simt_supported(dtype, head_dim, group);
  const bool mfma_ok = pkv::mfma_supported(dtype, head_dim, group);
  const bool fused = app.slot_mapping != nullptr;
  bool use_mfma;
  switch (impl) {
    case PKV_IMPL_AUTO:
      if (!simt_ok && !mfma_ok) return PKV_E_UNSUPPORTED;
      use_mfma = mfma_ok;
      break;
    case PKV_IMPL_SIMT:
      if (!simt_ok) return PKV_E_UNSUPPORTED;
      use_mfma = false;
      break;
    case PKV_IMPL_MFMA:
      if (!mfma_ok) return PKV_E_UNSUPPORTED;
      use_mfma = true;
      break;
    default: return PKV_E_UNSUPPORTED;
  }
  if (fused && !use_mfma) return PKV_E_UNSUPPORTED;  // the append is fused into the MFMA kernels only
  if (fp8 && !use_mfma) return PKV_E_UNSUPPORTED;    // FP8 pools: MFMA kernel
  if (fp8 && (!scale_ok(fp8->k) || !scale_ok(fp8->v))) return PKV_E_SHAPE;
  if (pre && (pre->num_items < 0 || pre->max_prefix_len < 0 || pre->max_prefix_len > max_context_len))
    return PKV_E_SHAPE;
  // no items or no prefix length: the call is the plain decode
  const bool prefixed = pre && pre->num_items > 0 && pre->max_prefix_len > 0;
  if (prefixed && (!use_mfma || fp8)) return PKV_E_UNSUPPORTED;  // shared prefixes: MFMA kernel, 16-bit pools
  if (num_seqs == 0) return PKV_OK;
  if (prefixed && (!pre->prefix_len || !pre->prefix_items)) return PKV_E_NULL;
  if (num_work < 0) return PKV_E_SHAPE;
  if (num_work > 0 && (!use_mfma || fp8)) return PKV_E_UNSUPPORTED;  // work lists: MFMA kernel, 16-bit pools
  if (num_work > 0 && !work) return PKV_E_NULL;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out) return PKV_E_NULL;
  if (fused && (!app.k_new || !app.v_new)) return PKV_E_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return PKV_E_SHAPE;
  if (fused && (!aligned16(app.k_new) || !aligned16(app.v_new))) return PKV_E_SHAPE;

  const Plan plan = make_plan(num_seqs, num_kv_heads, max_context_len, partition_tokens);
  const int32_t chunks = prefixed ? prefix_chunk_count(pre->max_prefix_len) : 0;
  const size_t need = workspace_for(num_seqs, num_q_heads, head_dim, plan, chunks);
  if (need > 0 && (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u)))
    return PKV_E_WORKSPACE;
  const int64_t items = static_cast<int64_t>(num_seqs) * plan.num_parts * num_kv_heads;
  if (items > INT_MAX) return PKV_E_SHAPE;
  if (prefixed && static_cast<int64_t>(pre->num_items) * num_kv_heads * chunks > INT_MAX) return PKV_E_SHAPE;

  pkv::DecodeParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k_cache = static_cast<const uint16_t*>(k_cache);
  p.v_cache = static_cast<const uint16_t*>(v_cache);
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.out = static_cast<uint16_t*>(out);
  p.part_o = nullptr;
  p.part_m = nullptr;
  p.part_l = nullptr;
  if (need > 0) {
    const size_t rows = static_cast<size_t>(num_seqs) * num_q_heads * (plan.num_parts + chunks);
    char* ws = static_cast<char*>(workspace);
    p.part_o = reinterpret_cast<float*>(ws);
    p.part_m = reinterpret_cast<float*>(ws + align256(rows * head_dim * sizeof(float)));
    p.part_l = reinterpret_cast<float*>(ws + align256(rows * head_dim * sizeof(float)) + align256(rows * sizeof(float)));
  }
  p.k_new = static_cast<const uint16_t*>(app.k_new);
  p.v_new = static_cast<const uint16_t*>(app.v_new);
  p.slot_mapping = app.slot_mapping;
  p.append_wgs = 0;  // set by the MFMA launcher for fused calls
  p.seq_order = num_work > 0 ? nullptr : seq_order;  // the work list carries the order

  p.num_seqs = num_seqs;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.num_blocks = num_blocks;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_context_len = max_context_len;
  p.part_tokens = plan.part_tokens;
  p.num_parts = plan.num_parts;
  pkv::DecodeExt x{};
  x.prefix_len = prefixed ? pre->prefix_len : nullptr;
  x.prefix_items = prefixed ? pre->prefix_items : nullptr;
  x.num_prefix_items = prefixed ? pre->num_items : 0;
  x.max_prefix_len = prefixed ? pre->max_prefix_len : 0;
  x.prefix_chunk = prefixed ? prefix_chunk_tokens(pre->max_prefix_len) : 0;
  x.prefix_chunks = chunks;
  x.prefix_wgs = 0;  // set by the MFMA launcher
  x.num_slots = plan.num_parts + chunks;
  x.work = num_work > 0 ? work : nullptr;
  x.num_work = num_work > 0 ? num_work : 0;
  p.scale_log2 = static_cast<float>(static_cast<double>(scale) * (fp8 ? fp8->k : 1.0) * kLog2e);
  p.out_scale = fp8 ? fp8->v : 1.f;
  // the fused FP8 append encodes x * (1 / scale), exactly as pkv_kv_append_fp8
  p.k_inv_scale = fp8 ? 1.f / fp8->k : 1.f;
  p.v_inv_scale = fp8 ? 1.f / fp8->v : 1.f;

  hipError_t e = fp8        ? pkv::launch_decode_fp8(p, dtype, stream)
                 : use_mfma ? pkv::launch_decode_mfma(p, x, dtype, stream)
                            : pkv::launch_decode_simt(p, dtype, stream);
  if (e != hipSuccess) return PKV_E_HIP;
  if (plan.num_parts + chunks > 1) {
    e = pkv::launch_merge(p, x, dtype, stream);
    if (e != hipSuccess) return PKV_E_HIP;
  }
  return PKV_OK;
}

}  // namespace

int pkv_paged_attn_decode_ex(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_tables, int32_t max_blocks_per_seq,
                             const int32_t* context_lens, int32_t max_context_len, float scale,
                             void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                             int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t dtype,
                             void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                             int32_t impl, const int32_t* seq_order, hipStream_t stream) {
  return decode_call(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, max_context_len, scale,
                     out, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, dtype, workspace,
                     workspace_bytes, partition_tokens, impl, FusedAppend{nullptr, nullptr, nullptr}, nullptr,
                     seq_order, stream);
}

int pkv_append_paged_attn_decode(const void* q, const void* k_new, const void* v_new,
                                 const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                 const int32_t* block_tables, int32_t max_blocks_per_seq,
                                 const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                                 int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                 int32_t block_size, int32_t num_blocks, int32_t dtype, void* workspace,
                                 size_t workspace_bytes, int32_t partition_tokens, const int32_t* seq_order,
                                 hipStream_t stream) {
  if (num_seqs > 0 && !slot_mapping) return PKV_E_NULL;
  return decode_call(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, max_context_len, scale,
                     out, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, dtype, workspace,
                     workspace_bytes, partition_tokens, PKV_IMPL_MFMA, FusedAppend{k_new, v_new, slot_mapping},
                     nullptr, seq_order, stream);
}

int pkv_paged_attn_decode(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_tables, int32_t max_blocks_per_seq,
                          const int32_t* context_lens, int32_t max_context_len, float scale,
                          void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                          int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t dtype,
                          void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return pkv_paged_attn_decode_ex(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                                  max_context_len, scale, out, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                  block_size, num_blocks, dtype, workspace, workspace_bytes, 0, PKV_IMPL_AUTO,
                                  nullptr, stream);
}

int pkv_paged_attn_decode_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                  const int32_t* block_tables, int32_t max_blocks_per_seq,
                                  const int32_t* context_lens, int32_t max_context_len, float scale, void* out,
                                  int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                  int32_t block_size, int32_t num_blocks, int32_t dtype, hipStream_t stream) {
  // the split plan's partial states need more than the scratch holds: refuse
  // before touching the device
  if (num_seqs > 0 && num_q_heads > 0 && num_kv_heads > 0 && head_dim > 0 && max_context_len > 0 &&
      num_q_heads % num_kv_heads == 0) {
    const Plan plan = make_plan(num_seqs, num_kv_heads, max_context_len, 0);
    if (workspace_for(num_seqs, num_q_heads, head_dim, plan) > pkv::kNoAllocScratchBytes) return PKV_E_WORKSPACE;
  }
  void* ws = nullptr;
  if (pkv::noalloc_scratch(&ws) != hipSuccess) return PKV_E_HIP;
  return pkv_paged_attn_decode_ex(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens,
                                  max_context_len, scale, out, num_seqs, num_q_heads, num_kv_heads, head_dim,
                                  block_size, num_blocks, dtype, ws, pkv::kNoAllocScratchBytes, 0, PKV_IMPL_AUTO,
                                  nullptr, stream);
}

int pkv_paged_prefill(const void* q, const void* k_cache, const void* v_cache, const int32_t* block_tables,
                      int32_t max_blocks_per_seq, const int32_t* context_lens, const int32_t* query_start,
                      int32_t num_tokens, int32_t max_query_len, int32_t max_context_len, float scale, void* out,
                      int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                      int32_t block_size, int32_t num_blocks, int32_t dtype, hipStream_t stream) {
  if (num_seqs < 0 || num_tokens < 0 || max_query_len < 0 || max_context_len < 0 || num_q_heads <= 0 ||
      num_kv_heads <= 0 || num_blocks <= 0 || max_blocks_per_seq <= 0)
    return PKV_E_SHAPE;
  if (num_q_heads % num_kv_heads) return PKV_E_SHAPE;
  if (static_cast<int64_t>(max_context_len) > static_cast<int64_t>(max_blocks_per_seq) * block_size)
    return PKV_E_SHAPE;
  if (!scale_ok(scale)) return PKV_E_SHAPE;
  if (!dtype_ok(dtype) || !block_size_ok(block_size) || !pkv::mfma_supported(dtype, head_dim, num_q_heads / num_kv_heads))
    return PKV_E_UNSUPPORTED;
  if (static_cast<int64_t>(num_blocks) * num_kv_heads * (block_size / 16) > INT_MAX) return PKV_E_SHAPE;
  if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !query_start || !out) return PKV_E_NULL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(out)) return PKV_E_SHAPE;
  pkv::PrefillParams p;
  p.q = static_cast<const uint16_t*>(q);
  p.k_cache = static_cast<const uint16_t*>(k_cache);
  p.v_cache = static_cast<const uint16_t*>(v_cache);
  p.block_tables = block_tables;
  p.context_lens = context_lens;
  p.query_start = query_start;
  p.out = static_cast<uint16_t*>(out);
  p.num_seqs = num_seqs;
  p.num_tokens = num_tokens;
  p.num_q_heads = num_q_heads;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.block_size = block_size;
  p.num_blocks = num_blocks;
  p.max_blocks_per_seq = max_blocks_per_seq;
  p.max_context_len = max_context_len;
  p.max_query_len = max_query_len;
  p.chunks = 0;
  p.scale_log2 = static_cast<float>(static_cast<double>(scale) * kLog2e);
  return pkv::launch_prefill_mfma(p, dtype, stream) == hipSuccess ? PKV_OK : PKV_E_HIP;
}

int pkv_kv_append_fp8(const void* k, const void* v, const int64_t* slot_mapping, int32_t num_tokens,
                      void* k_cache, void* v_cache, int32_t num_blocks, int32_t block_size, int32_t num_kv_heads,
                      int32_t head_dim, int32_t src_dtype, float k_scale, float v_scale, hipStream_t stream) {
  if (num_tokens < 0 || num_blocks <= 0 || num_kv_heads <= 0) return PKV_E_SHAPE;
  if (!dtype_ok(src_dtype) || !block_size_ok(block_size) || head_dim <= 0 || head_dim % 8 || head_dim > 512)
    return PKV_E_UNSUPPORTED;
  if (!scale_ok(k_scale) || !scale_ok(v_scale)) return PKV_E_SHAPE;
  if (num_tokens == 0) return PKV_OK;
  if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PKV_E_NULL;
  if (!aligned16(k) || !aligned16(v) || !aligned16(k_cache) || !aligned16(v_cache)) return PKV_E_SHAPE;
  if (static_cast<int64_t>(num_tokens) * num_kv_heads * (head_dim / 8) > static_cast<int64_t>(INT_MAX) * 256)
    return PKV_E_SHAPE;
  pkv::AppendFp8Params p;
  p.k = static_cast<const uint16_t*>(k);
  p.v = static_cast<const uint16_t*>(v);
  p.slot_mapping = slot_mapping;
  p.k_cache = static_cast<uint8_t*>(k_cache);
  p.v_cache = static_cast<uint8_t*>(v_cache);
  p.k_inv_scale = 1.f / k_scale;
  p.v_inv_scale = 1.f / v_scale;
  p.num_tokens = num_tokens;
  p.num_blocks = num_blocks;
  p.block_size = block_size;
  p.num_kv_heads = num_kv_heads;
  p.head_dim = head_dim;
  p.src_fp16 = src_dtype == PKV_FP16;
  return pkv::launch_kv_append_fp8(p, stream) == hipSuccess ? PKV_OK : PKV_E_HIP;
}

int pkv_paged_attn_decode_fp8(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, int32_t max_blocks_per_seq,
                              const int32_t* context_lens, int32_t max_context_len, float scale, float k_scale,
                              float v_scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                              int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                              int32_t dtype, void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                              const int32_t* seq_order, hipStream_t stream) {
  const Fp8Scales sc{k_scale, v_scale};
  return decode_call(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, max_context_len, scale,
                     out, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, dtype, workspace,
                     workspace_bytes, partition_tokens, PKV_IMPL_MFMA, FusedAppend{nullptr, nullptr, nullptr}, &sc,
                     seq_order, stream);
}

int pkv_append_paged_attn_decode_fp8(const void* q, const void* k_new, const void* v_new,
                                     const int64_t* slot_mapping, void* k_cache, void* v_cache,
                                     const int32_t* block_tables, int32_t max_blocks_per_seq,
                                     const int32_t* context_lens, int32_t max_context_len, float scale,
                                     float k_scale, float v_scale, void* out, int32_t num_seqs, int32_t num_q_heads,
                                     int32_t num_kv_heads, int32_t head_dim, int32_t block_size, int32_t num_blocks,
                                     int32_t dtype, void* workspace, size_t workspace_bytes, int32_t partition_tokens,
                                     const int32_t* seq_order, hipStream_t stream) {
  if (num_seqs > 0 && !slot_mapping) return PKV_E_NULL;
  const Fp8Scales sc{k_scale, v_scale};
  return decode_call(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, max_context_len, scale,
                     out, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, dtype, workspace,
                     workspace_bytes, partition_tokens, PKV_IMPL_MFMA, FusedAppend{k_new, v_new, slot_mapping}, &sc,
                     seq_order, stream);
}

int pkv_decode_prefix_plan(const int32_t* block_tables, int32_t max_blocks_per_seq, const int32_t* context_lens,
                           int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                           int32_t block_size, int32_t* prefix_len, int32_t* prefix_items, int32_t max_items,
                           int32_t* num_items, int32_t* max_prefix_len) {
  if (num_seqs < 0 || max_blocks_per_seq <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || max_items < 0)
    return PKV_E_SHAPE;
  if (num_q_heads % num_kv_heads) return PKV_E_SHAPE;
  if (!block_size_ok(block_size)) return PKV_E_UNSUPPORTED;
  const int32_t group = num_q_heads / num_kv_heads;
  if (!pkv::mfma_supported(PKV_BF16, head_dim, group)) return PKV_E_UNSUPPORTED;
  if (!num_items || !max_prefix_len) return PKV_E_NULL;
  *num_items = 0;
  *max_prefix_len = 0;
  if (num_seqs == 0) return PKV_OK;
  if (!block_tables || !context_lens || !prefix_len || (max_items > 0 && !prefix_items)) return PKV_E_NULL;
  const int32_t per_item = pkv::prefix_members_per_item(head_dim, group);
  const size_t row = static_cast<size_t>(max_blocks_per_seq);

  // full[i]: sequence i's blocks that are full before its last position (the
  // only ones it may share: the token of this step goes after them)
  std::vector<int32_t> full(num_seqs, 0), cand;
  for (int32_t i = 0; i < num_seqs; ++i) {
    prefix_len[i] = 0;
    const int64_t L = context_lens[i];
    if (L < 2 || L > static_cast<int64_t>(max_blocks_per_seq) * block_size) continue;
    full[i] = static_cast<int32_t>((L - 1) / block_size);
    if (full[i] > 0) cand.push_back(i);
  }
  // leading blocks two sequences have in common (within both full ranges)
  auto common = [&](int32_t a, int32_t b) {
    const int32_t n = std::min(full[a], full[b]);
    const int32_t* ra = block_tables + static_cast<size_t>(a) * row;
    const int32_t* rb = block_tables + static_cast<size_t>(b) * row;
    int32_t k = 0;
    while (k < n && ra[k] == rb[k]) ++k;
    return k;
  };
  // rows in lexicographic order of their full blocks, a row that is a prefix
  // of another after it (so sequences with long common prefixes are neighbours
  // and each run starts with its longest row)
  std::stable_sort(cand.begin(), cand.end(), [&](int32_t a, int32_t b) {
    const int32_t k = common(a, b);
    if (k < full[a] && k < full[b])
      return block_tables[static_cast<size_t>(a) * row + k] < block_tables[static_cast<size_t>(b) * row + k];
    return full[a] > full[b];
  });
  // items: a reference and the following rows that share at least its first
  // block, up to per_item members; an item of one member is dropped
  int32_t items = 0, longest = 0;
  size_t i = 0;
  std::vector<int32_t> mem, lim;
  while (i < cand.size()) {
    const int32_t ref = cand[i];
    mem.assign(1, ref);
    lim.assign(1, 0);
    size_t j = i + 1;
    for (; j < cand.size() && static_cast<int32_t>(mem.size()) < per_item; ++j) {
      const int32_t c = common(cand[j], ref);
      if (c < 1) break;
      mem.push_back(cand[j]);
      lim.push_back(c);
    }
    i = j;
    if (mem.size() < 2) continue;
    if (items >= max_items) return PKV_E_SHAPE;
    lim[0] = *std::max_element(lim.begin() + 1, lim.end());
    int32_t* out = prefix_items + static_cast<size_t>(items) * 16;
    for (int32_t k = 0; k < 16; ++k) out[k] = k < static_cast<int32_t>(mem.size()) ? mem[k] : -1;
    for (size_t k = 0; k < mem.size(); ++k) {
      prefix_len[mem[k]] = lim[k] * block_size;
      longest = std::max(longest, lim[k] * block_size);
    }
    ++items;
  }
  *num_items = items;
  *max_prefix_len = longest;
  return PKV_OK;
}

int pkv_paged_attn_decode_prefix(const void* q, const void* k_new, const void* v_new, const int64_t* slot_mapping,
                                 void* k_cache, void* v_cache, const int32_t* block_tables,
                                 int32_t max_blocks_per_seq, const int32_t* context_lens, int32_t max_context_len,
                                 float scale, void* out, int32_t num_seqs, int32_t num_q_heads, int32_t num_kv_heads,
                                 int32_t head_dim, int32_t block_size, int32_t num_blocks, int32_t dtype,
                                 const int32_t* prefix_len, const int32_t* prefix_items, int32_t num_prefix_items,
                                 int32_t max_prefix_len, void* workspace, size_t workspace_bytes,
                                 int32_t partition_tokens, const int32_t* seq_order, const int32_t* work,
                                 int32_t num_work, hipStream_t stream) {
  const PrefixDesc pre{prefix_len, prefix_items, num_prefix_items, max_prefix_len};
  return decode_call(q, k_cache, v_cache, block_tables, max_blocks_per_seq, context_lens, max_context_len, scale,
                     out, num_seqs, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, dtype, workspace,
                     workspace_bytes, partition_tokens, PKV_IMPL_MFMA, FusedAppend{k_new, v_new, slot_mapping},
                     nullptr, seq_order, stream, &pre, work, num_work);
}

}  // extern "C"
