// C ABI of libindexpool: argument checks, workspace carving and kernel dispatch.
// Every check that the host can make happens before anything is enqueued.
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "../../include/indexpool.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_err;

ip_status fail(ip_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return st;
}

ip_status device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return IP_OK;
  return fail(IP_EDEVICE, "%s: launch failed: %s", what, hipGetErrorString(e));
}

struct Hook {
  hipEvent_t start = nullptr, stop = nullptr;
};
thread_local Hook g_hook[ip::K_LAST + 1];   // armed events per kernel id

constexpr int64_t kMaxTokens = int64_t(1) << 31;   // int32 token positions
constexpr size_t kScoreBudget = size_t(256) << 20;  // score workspace per row chunk
#ifndef IP_ATTN_WG
#define IP_ATTN_WG 128
#endif
constexpr int kComputeUnits = 256;                     // gfx950: 8 dies x 32
constexpr int kAttnWorkgroups = IP_ATTN_WG;               // split decode attention up to this many workgroups

ip_status check_seqs(const ip_seqs* s, const char* fn) {
  if (!s) return fail(IP_EINVAL, "%s: seqs is NULL", fn);
  if (s->batch < 1) return fail(IP_EINVAL, "%s: batch must be >= 1 (got %d)", fn, s->batch);
  if (!s->seq_lens) return fail(IP_EINVAL, "%s: seqs->seq_lens is NULL", fn);
  if (s->max_seq_len < 1 || s->max_seq_len >= kMaxTokens)
    return fail(IP_EINVAL, "%s: max_seq_len out of range (got %d)", fn, s->max_seq_len);
  if (s->page_table) {
    if (s->page_tokens < 4 || s->page_tokens % 4)
      return fail(IP_EINVAL, "%s: page_tokens must be a positive multiple of 4 (got %d)", fn, s->page_tokens);
    if (s->max_pages < 1) return fail(IP_EINVAL, "%s: max_pages must be >= 1", fn);
    if ((int64_t)s->max_pages * s->page_tokens < s->max_seq_len)
      return fail(IP_EINVAL, "%s: max_pages * page_tokens < max_seq_len", fn);
  } else {
    if (s->seq_stride < s->max_seq_len || s->seq_stride % 4)
      return fail(IP_EINVAL, "%s: seq_stride must be a multiple of 4 and >= max_seq_len (got %lld)", fn,
                  (long long)s->seq_stride);
  }
  return IP_OK;
}

ip::Layout layout_of(const ip_seqs* s) {
  ip::Layout L;
  L.seq_lens = s->seq_lens;
  L.page_table = s->page_table;
  L.max_pages = s->max_pages;
  L.page_tokens = s->page_tokens;
  L.seq_stride = s->seq_stride;
  return L;
}

int elem_bytes(int dt) { return dt == IP_F32 ? 4 : dt == IP_BF16 ? 2 : 1; }

ip_status check_cache(const ip_cache* c, const char* fn, const char* name) {
  if (!c) return fail(IP_EINVAL, "%s: %s is NULL", fn, name);
  if (!c->data) return fail(IP_EINVAL, "%s: %s->data is NULL", fn, name);
  if (c->dtype < IP_F32 || c->dtype > IP_FP8_E4M3FN) return fail(IP_EUNSUPPORTED, "%s: %s has an unknown dtype", fn, name);
  if (c->row_dim < 1) return fail(IP_EINVAL, "%s: %s->row_dim must be >= 1", fn, name);
  if (c->row_stride % 16 || c->row_stride < (int64_t)c->row_dim * elem_bytes(c->dtype))
    return fail(IP_EINVAL, "%s: %s->row_stride must be a multiple of 16 covering a row", fn, name);
  if ((reinterpret_cast<uintptr_t>(c->data) & 15) != 0) return fail(IP_EINVAL, "%s: %s->data must be 16-byte aligned", fn, name);
  if (c->dtype == IP_FP8_E4M3FN && !c->scale) return fail(IP_EINVAL, "%s: %s->scale is required for FP8", fn, name);
  return IP_OK;
}

// Score workspace plan shared by the size query and the call: per-row counters
// of the fused selection, group maxima, then (unless the caller keeps the scores)
// the scores of one pass of rows.
struct ScorePlan {
  int64_t ld, gld;     // floats per score row / per group-maximum row
  int max_blocks;      // eligible blocks bound
  int rows_per_pass;   // query rows per pass
  int max_lists;       // per-wave candidate lists per row (0: rows too long for them)
  int wg_lists;        // else per-workgroup lists per row (1M-token rows), or 0
  size_t count_bytes, ack_bytes, gm_bytes, list_bytes, score_bytes, total;
};

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

ScorePlan score_plan(const ip_seqs* s, int n_q, bool scores_given) {
  ScorePlan p;
  p.max_blocks = (s->max_seq_len - 1) / 4;          // j < b_q <= (max_seq_len - 1) / 4
  p.ld = index_scores_ld(s->max_seq_len);
  p.gld = p.ld / 16;
  if (scores_given) {
    p.rows_per_pass = n_q;
  } else {
    const size_t per_row = (size_t)p.ld * 4;
    p.rows_per_pass = (int)std::max<size_t>(1, std::min<size_t>(n_q, kScoreBudget / per_row));
  }
  p.count_bytes = align256((size_t)p.rows_per_pass * 4);
  p.gm_bytes = align256((size_t)p.rows_per_pass * p.gld * 4);
  // decode-shaped calls (fewer than 64 rows): 16-entry lists of each 128-block wave
  // of a row, when a row has at most 256 of them (the selection merges them in LDS)
  const int waves = 8 * (int)((std::max(1, p.max_blocks) + 1023) / 1024);
  p.max_lists = waves <= 256 && n_q < 64 ? waves : 0;
  // longer decode rows: one 16-entry list per 8-wave workgroup, up to 256 of them
  p.wg_lists = !p.max_lists && n_q < 64 && waves / 8 <= 256 ? waves / 8 : 0;
  p.list_bytes = align256((size_t)p.rows_per_pass * (p.max_lists + p.wg_lists) * (16 * 8 + 8));
  p.ack_bytes = p.max_lists ? align256((size_t)p.rows_per_pass * 12) : 0;
  p.score_bytes = scores_given ? 0 : align256((size_t)p.rows_per_pass * p.ld * 4);
  p.total = p.count_bytes + p.ack_bytes + p.gm_bytes + p.list_bytes + p.score_bytes;
  return p;
}

struct AttnPlan {
  int n_split, blocks_per_split;
  size_t bytes;
};

AttnPlan attn_plan(int n_q, int n_heads, int dv, int top_k, int q_dtype) {
  AttnPlan p;
  p.n_split = 1;
  p.blocks_per_split = top_k;
  if (q_dtype == IP_BF16) {
    // one workgroup per (row, split) covering all 64 heads; splits add workgroups
    // for small batches at the price of (O, m, l) partials (64 KB per split)
    const int nsub = (top_k + 15) / 16;                 // 64-token sub-tiles
    const int want = (kAttnWorkgroups + n_q - 1) / std::max(1, n_q);
    const int ns = std::max(1, std::min(want, std::min(nsub, 64)));
    const int sub_per = std::min((nsub + ns - 1) / ns, 32);   // <= 512 blocks per split
    p.blocks_per_split = sub_per * 16;
    p.n_split = (top_k + p.blocks_per_split - 1) / p.blocks_per_split;
    // long splits run one pipelined workgroup per compute unit: halve them while a
    // launch has fewer units than the chip has compute units and the halves stay
    // long enough for the pipelined kernel
    while ((int64_t)p.n_split * n_q < kComputeUnits && p.blocks_per_split >= 2 * ip::PIPE_MIN_BLOCKS) {
      p.blocks_per_split /= 2;
      p.n_split = (top_k + p.blocks_per_split - 1) / p.blocks_per_split;
    }
  }
  // bf16 partial O, then fp32 (m, l) pairs
  p.bytes = p.n_split > 1 ? (size_t)n_q * p.n_split * n_heads * ((size_t)dv * 2 + 8) : 0;
  return p;
}

}  // namespace

namespace ip {
bool hook_take(int id, hipEvent_t* start, hipEvent_t* stop) {
  if (id < 1 || id > K_LAST || !g_hook[id].start) return false;
  *start = g_hook[id].start;
  *stop = g_hook[id].stop;
  g_hook[id] = Hook{};
  return true;
}
}  // namespace ip

extern "C" {

const char* ip_last_error(void) { return g_err.c_str(); }
const char* ip_version(void) { return "0.1.0"; }

ip_status ip_phase_stamps(void* host, size_t bytes) {
  if (!host) return fail(IP_EINVAL, "ip_phase_stamps: host is NULL");
  if (!ip::phase_stamps(host, bytes))
    return fail(IP_EUNSUPPORTED, "ip_phase_stamps: the library was built without IP_PHASE_STAMPS");
  return IP_OK;
}

ip_status ip_time_next_launch(int32_t kernel_id, hipEvent_t start, hipEvent_t stop) {
  if (kernel_id == 0 && !start && !stop) {
    for (auto& h : g_hook) h = Hook{};
    return IP_OK;
  }
  if (kernel_id < ip::K_COMPRESS || kernel_id > ip::K_LAST)
    return fail(IP_EINVAL, "ip_time_next_launch: unknown kernel id %d", kernel_id);
  if (!start != !stop) return fail(IP_EINVAL, "ip_time_next_launch: pass both events or neither");
  g_hook[kernel_id].start = start;
  g_hook[kernel_id].stop = stop;
  return IP_OK;
}

int64_t index_scores_ld(int32_t max_seq_len) {
  // whole scoring tiles, so every scoring workgroup stores inside its row and the
  // selection's vector reads stay inside the row
  const int64_t n = std::max<int64_t>(1, max_seq_len / 4);
  return (n + ip::SCORE_TILE - 1) / ip::SCORE_TILE * ip::SCORE_TILE;
}

// ------------------------------------------------------------------ IndexPool
ip_status indexpool_compress(const ip_seqs* seqs, const int32_t* block_begin, int32_t max_blocks,
                             const ip_cache* keys, const float* logits, const ip_cache* pooled,
                             hipStream_t stream) {
  const char* fn = "indexpool_compress";
  if (ip_status st = check_seqs(seqs, fn)) return st;
  if (ip_status st = check_cache(keys, fn, "keys")) return st;
  if (ip_status st = check_cache(pooled, fn, "pooled")) return st;
  if (!logits) return fail(IP_EINVAL, "%s: logits is NULL", fn);
  if (keys->dtype != pooled->dtype || keys->row_dim != pooled->row_dim)
    return fail(IP_EINVAL, "%s: keys and pooled must share dtype and row_dim", fn);
  ip::CompressArgs a;
  a.L = layout_of(seqs);
  a.batch = seqs->batch;
  a.block_begin = block_begin;
  a.max_blocks = max_blocks > 0 ? max_blocks : seqs->max_seq_len / 4;
  a.keys = (const uint8_t*)keys->data;
  a.key_stride = keys->row_stride;
  a.key_scale = keys->scale;
  a.logits = logits;
  a.out = (uint8_t*)pooled->data;
  a.out_stride = pooled->row_stride;
  a.out_scale = pooled->scale;
  a.dim = keys->row_dim;
  if (seqs->batch > 65535) return fail(IP_EUNSUPPORTED, "%s: batch > 65535", fn);
  if (keys->dtype == IP_FP8_E4M3FN) {
    if (keys->row_dim != 128) return fail(IP_EUNSUPPORTED, "%s: FP8 keys need row_dim 128 (got %d)", fn, keys->row_dim);
    return device_status(ip::launch_compress_fp8(a, stream), fn);
  }
  if (keys->dtype == IP_F32) {
    if (keys->row_dim > 256 || keys->row_dim % 4)
      return fail(IP_EUNSUPPORTED, "%s: F32 keys need row_dim <= 256 and a multiple of 4", fn);
    return device_status(ip::launch_compress_f32(a, stream), fn);
  }
  return fail(IP_EUNSUPPORTED, "%s: keys must be FP8 or F32", fn);
}

// ------------------------------------------------------------------ decode append
}  // extern "C"

// Checks the append arguments and fills `a` (no launch).
static ip_status build_append(const char* fn, const ip_seqs* seqs, const void* kv_new, const ip_cache* kv,
                              const void* v_new, const ip_cache* v, const void* key_new, int32_t key_dtype,
                              const ip_cache* keys, const float* logit_new, float* logits, const ip_cache* pooled,
                              ip::AppendArgs& a) {
  if (ip_status st = check_seqs(seqs, fn)) return st;
  if (ip_status st = check_cache(kv, fn, "kv")) return st;
  if (!kv_new) return fail(IP_EINVAL, "%s: kv_new must not be NULL", fn);
  const bool idx = keys != nullptr;              // NULL keys: a layer without indexer state
  if (idx) {
    if (ip_status st = check_cache(keys, fn, "keys")) return st;
    if (ip_status st = check_cache(pooled, fn, "pooled")) return st;
    if (!key_new || !logit_new || !logits)
      return fail(IP_EINVAL, "%s: key_new, logit_new and logits must not be NULL when keys are given", fn);
  } else if (key_new || logit_new || logits || pooled) {
    return fail(IP_EINVAL, "%s: without keys, key_new, logit_new, logits and pooled must be NULL", fn);
  }
  if (v) {
    if (ip_status st = check_cache(v, fn, "v")) return st;
    if (!v_new) return fail(IP_EINVAL, "%s: v_new is NULL while v is given", fn);
  }
  const bool kv8 = kv->dtype == IP_FP8_E4M3FN;
  if (v && v->dtype == IP_FP8_E4M3FN) return fail(IP_EUNSUPPORTED, "%s: a separate v cache must be BF16 or F32", fn);
  if (kv8 && (v || kv->row_dim % 4 || kv->row_dim > 1024))
    return fail(IP_EUNSUPPORTED, "%s: an FP8 kv cache needs v = NULL and row_dim a multiple of 4, <= 1024", fn);
  if (kv8 && ((uintptr_t)kv_new & 7))
    return fail(IP_EINVAL, "%s: kv_new must be 8-byte aligned", fn);
  const int kv_bytes = kv8 ? 0 : kv->row_dim * elem_bytes(kv->dtype);
  const int v_bytes = v ? v->row_dim * elem_bytes(v->dtype) : 0;
  if (kv_bytes % 16 || v_bytes % 16) return fail(IP_EUNSUPPORTED, "%s: kv / v rows must be whole 16-byte chunks", fn);
  if (idx) {
    if (keys->dtype != pooled->dtype || keys->row_dim != pooled->row_dim)
      return fail(IP_EINVAL, "%s: keys and pooled must share dtype and row_dim", fn);
    if (keys->dtype == IP_FP8_E4M3FN) {
      if (keys->row_dim != 128) return fail(IP_EUNSUPPORTED, "%s: FP8 keys need row_dim 128 (got %d)", fn, keys->row_dim);
      if (key_dtype != IP_BF16 && key_dtype != IP_F32) return fail(IP_EUNSUPPORTED, "%s: key_new must be BF16 or F32", fn);
    } else if (keys->dtype == IP_F32) {
      if (keys->row_dim > 256) return fail(IP_EUNSUPPORTED, "%s: F32 keys need row_dim <= 256", fn);
      if (key_dtype != IP_F32) return fail(IP_EUNSUPPORTED, "%s: F32 keys take an F32 key_new", fn);
    } else {
      return fail(IP_EUNSUPPORTED, "%s: keys must be FP8 or F32", fn);
    }
  }
  if (seqs->batch > 65535) return fail(IP_EUNSUPPORTED, "%s: batch > 65535", fn);
  a.L = layout_of(seqs);
  a.batch = seqs->batch;
  a.kv_new = (const uint8_t*)kv_new;
  a.kv = (uint8_t*)kv->data;
  a.kv_stride = kv->row_stride;
  a.kv_row_bytes = kv_bytes;
  a.kv_scale = kv8 ? kv->scale : nullptr;
  a.kv_dim = kv->row_dim;
  a.v_new = (const uint8_t*)v_new;
  a.v = v ? (uint8_t*)v->data : nullptr;
  a.v_stride = v ? v->row_stride : 0;
  a.v_row_bytes = v_bytes;
  a.key_new = key_new;
  a.key_bf16 = key_dtype == IP_BF16;
  a.keys = idx ? (uint8_t*)keys->data : nullptr;
  a.key_stride = idx ? keys->row_stride : 0;
  a.key_scale = idx && keys->dtype == IP_FP8_E4M3FN ? keys->scale : nullptr;
  a.dim = idx ? keys->row_dim : 0;
  a.logit_new = logit_new;
  a.logits = logits;
  a.pooled = idx ? (uint8_t*)pooled->data : nullptr;
  a.pooled_stride = idx ? pooled->row_stride : 0;
  a.pooled_scale = idx && keys->dtype == IP_FP8_E4M3FN ? pooled->scale : nullptr;
  return IP_OK;
}

extern "C" {

ip_status indexpool_append(const ip_seqs* seqs, const void* kv_new, const ip_cache* kv, const void* v_new,
                           const ip_cache* v, const void* key_new, int32_t key_dtype, const ip_cache* keys,
                           const float* logit_new, float* logits, const ip_cache* pooled, hipStream_t stream) {
  const char* fn = "indexpool_append";
  ip::AppendArgs a;
  if (ip_status st = build_append(fn, seqs, kv_new, kv, v_new, v, key_new, key_dtype, keys, logit_new, logits,
                                  pooled, a))
    return st;
  return device_status(ip::launch_append(a, stream), fn);
}

// ------------------------------------------------------------------ indexer + top-k
size_t index_score_topk_workspace_bytes(const ip_seqs* seqs, int32_t n_q, int32_t top_k,
                                        int32_t scores_given) {
  if (!seqs || n_q < 1 || top_k < 1 || seqs->max_seq_len < 1) return 0;
  return score_plan(seqs, n_q, scores_given != 0).total;
}

}  // extern "C"

// The checks of an indexer call (index_score_topk and the calls built on it).
static ip_status score_check(const char* fn, const ip_seqs* seqs, int32_t n_q, const int32_t* q_seq,
                             const void* q_idx, int32_t q_dtype, int32_t n_heads, int32_t head_dim,
                             const float* gates, const ip_cache* pooled, int32_t top_k, int32_t* out_idx) {
  if (ip_status st = check_seqs(seqs, fn)) return st;
  if (ip_status st = check_cache(pooled, fn, "pooled")) return st;
  if (n_q < 1) return fail(IP_EINVAL, "%s: n_q must be >= 1", fn);
  if (!q_idx || !gates || !out_idx) return fail(IP_EINVAL, "%s: q_idx, gates and out_idx are required", fn);
  if (top_k < 1 || top_k > 2048) return fail(IP_EUNSUPPORTED, "%s: top_k must be in 1..2048 (got %d)", fn, top_k);
  if (!q_seq && n_q > seqs->batch) return fail(IP_EINVAL, "%s: q_seq is NULL but n_q > batch", fn);
  if (pooled->row_dim != head_dim) return fail(IP_EINVAL, "%s: head_dim %d != pooled row_dim %d", fn, head_dim, pooled->row_dim);
  if (pooled->dtype == IP_FP8_E4M3FN) {
    if (q_dtype != IP_BF16 || n_heads != 32 || head_dim != 128)
      return fail(IP_EUNSUPPORTED, "%s: FP8 keys need BF16 queries with 32 heads x 128 dims", fn);
  } else if (pooled->dtype == IP_F32) {
    if (q_dtype != IP_F32 || n_heads < 1 || n_heads > 64 || head_dim < 1 || n_heads * head_dim > 4096)
      return fail(IP_EUNSUPPORTED, "%s: F32 keys need F32 queries with n_heads <= 64 and n_heads*head_dim <= 4096", fn);
  } else {
    return fail(IP_EUNSUPPORTED, "%s: pooled keys must be FP8 or F32", fn);
  }
  return IP_OK;
}

// The scoring launch's arguments for rows [row0, row0 + nr) over the workspace ws
// carved by `plan` (counters, group maxima, lists, then scores unless given).
static ip::ScoreArgs score_args(const ip_seqs* seqs, const ScorePlan& plan, int row0, int nr, const int32_t* q_seq,
                                const int32_t* q_pos, const void* q_idx, int32_t n_heads, int32_t head_dim,
                                const float* gates, const ip_cache* pooled, int32_t top_k, int32_t* out_idx,
                                float* scores, void* ws, const ip::AppendArgs* append) {
  int32_t* count = (int32_t*)ws;
  uint32_t* ack = plan.ack_bytes ? (uint32_t*)((char*)ws + plan.count_bytes) : nullptr;
  float* gm = (float*)((char*)ws + plan.count_bytes + plan.ack_bytes);
  char* lists = (char*)ws + plan.count_bytes + plan.ack_bytes + plan.gm_bytes;
  float* score_buf = scores ? scores : (float*)(lists + plan.list_bytes);
  ip::ScoreArgs sa{};
  sa.L = layout_of(seqs);
  sa.row0 = row0;
  sa.n_rows = nr;
  sa.q_seq = q_seq;
  sa.q_pos = q_pos;
  sa.q = q_idx;
  sa.gates = gates;
  sa.keys = (const uint8_t*)pooled->data;
  sa.key_stride = pooled->row_stride;
  sa.key_scale = pooled->scale;
  // the kernels index scores, maxima and counters by (r - row0)
  sa.scores = scores ? score_buf + (int64_t)row0 * plan.ld : score_buf;
  sa.ld = plan.ld;
  sa.gm = gm;
  sa.gld = plan.gld;
  sa.heads = n_heads;
  sa.dim = head_dim;
  sa.max_blocks = plan.max_blocks;
  sa.top_k = top_k;
  sa.out = out_idx;
  sa.count = count;
  sa.ack = ack;
  sa.scores_own = scores == nullptr;
  sa.max_lists = plan.max_lists;
  sa.wg_lists = plan.wg_lists;
  const int lpr = plan.max_lists + plan.wg_lists;   // one of the two is 0
  sa.lists = lpr ? (uint64_t*)lists : nullptr;
  sa.lists_meta = lpr ? (uint2*)(lists + (size_t)plan.rows_per_pass * lpr * 16 * 8) : nullptr;
  sa.with_append = append && row0 == 0;
  if (sa.with_append) sa.append = *append;
  sa.fuse = 0;
  sa.fuse = pooled->dtype == IP_FP8_E4M3FN && ip::score_fuses_select(sa);
  return sa;
}

// index_score_topk, optionally with a decode append fused into the first scoring
// launch (FP8 keys) or launched just before it (F32 keys).
static ip_status score_topk_impl(const char* fn, const ip_seqs* seqs, int32_t n_q, const int32_t* q_seq,
                                 const int32_t* q_pos, const void* q_idx, int32_t q_dtype, int32_t n_heads,
                                 int32_t head_dim, const float* gates, const ip_cache* pooled, int32_t top_k,
                                 int32_t* out_idx, float* scores, void* ws, size_t ws_bytes, hipStream_t stream,
                                 const ip::AppendArgs* append) {
  if (ip_status st = score_check(fn, seqs, n_q, q_seq, q_idx, q_dtype, n_heads, head_dim, gates, pooled, top_k,
                                 out_idx))
    return st;
  const bool fp8 = pooled->dtype == IP_FP8_E4M3FN;
  const ScorePlan plan = score_plan(seqs, n_q, scores != nullptr);
  if (!ws || ws_bytes < plan.total)
    return fail(IP_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, plan.total, ws ? ws_bytes : 0);
  if (((uintptr_t)ws & 255) != 0) return fail(IP_EINVAL, "%s: ws must be 256-byte aligned", fn);

  if (append && !fp8) {
    if (ip_status st = device_status(ip::launch_append(*append, stream), fn)) return st;
    append = nullptr;
  }
  // rows that fit one register-resident chunk whose padding the score rows cover
  // take the chunk select (no group maxima needed); others the whole-row select
  const int chunk = ip::topk_chunk_size(std::max(1, plan.max_blocks));
  const bool chunk_select = chunk > 0 && chunk <= plan.ld;
  for (int row0 = 0; row0 < n_q; row0 += plan.rows_per_pass) {
    const int nr = std::min(plan.rows_per_pass, n_q - row0);
    ip::ScoreArgs sa = score_args(seqs, plan, row0, nr, q_seq, q_pos, q_idx, n_heads, head_dim, gates, pooled,
                                  top_k, out_idx, scores, ws, append);
    if (!sa.fuse && chunk_select) sa.gm = nullptr;
    ip_status st = device_status(fp8 ? ip::launch_score_fp8_bf16(sa, stream) : ip::launch_score_f32(sa, stream), fn);
    if (st) return st;
    if (sa.fuse) continue;
    if (chunk_select) {
      ip::TopkArgs ka{};
      ka.L = sa.L;
      ka.row0 = row0;
      ka.n_rows = nr;
      ka.q_seq = q_seq;
      ka.q_pos = q_pos;
      ka.scores = sa.scores;
      ka.ld = plan.ld;
      ka.top_k = top_k;
      ka.out = out_idx;
      ka.n_chunks = 1;
      ka.chunk = chunk;
      st = device_status(ip::launch_topk(ka, stream), fn);
      if (st) return st;
      continue;
    }
    ip::SelectArgs ta;
    ta.L = sa.L;
    ta.row0 = row0;
    ta.n_rows = nr;
    ta.q_seq = q_seq;
    ta.q_pos = q_pos;
    ta.scores = sa.scores;
    ta.ld = plan.ld;
    ta.gm = sa.gm;
    ta.gld = plan.gld;
    ta.top_k = top_k;
    ta.out = out_idx;
    st = device_status(ip::launch_select(ta, stream), fn);
    if (st) return st;
  }
  return IP_OK;
}

extern "C" {

ip_status index_score_topk(const ip_seqs* seqs, int32_t n_q, const int32_t* q_seq,
                           const int32_t* q_pos, const void* q_idx, int32_t q_dtype,
                           int32_t n_heads, int32_t head_dim, const float* gates,
                           const ip_cache* pooled, int32_t top_k, int32_t* out_idx,
                           float* scores, void* ws, size_t ws_bytes, hipStream_t stream) {
  return score_topk_impl("index_score_topk", seqs, n_q, q_seq, q_pos, q_idx, q_dtype, n_heads, head_dim, gates,
                         pooled, top_k, out_idx, scores, ws, ws_bytes, stream, nullptr);
}

ip_status indexpool_decode_index(const ip_seqs* seqs, const void* kv_new, const ip_cache* kv, const void* v_new,
                                 const ip_cache* v, const void* key_new, int32_t key_dtype, const ip_cache* keys,
                                 const float* logit_new, float* logits, const ip_cache* pooled, const void* q_idx,
                                 int32_t q_dtype, int32_t n_heads, int32_t head_dim, const float* gates,
                                 int32_t top_k, int32_t* out_idx, float* scores, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  const char* fn = "indexpool_decode_index";
  if (!keys) return fail(IP_EINVAL, "%s: keys are required (the scoring reads the pooled keys)", fn);
  ip::AppendArgs a;
  if (ip_status st = build_append(fn, seqs, kv_new, kv, v_new, v, key_new, key_dtype, keys, logit_new, logits,
                                  pooled, a))
    return st;
  return score_topk_impl(fn, seqs, seqs->batch, nullptr, nullptr, q_idx, q_dtype, n_heads, head_dim, gates, pooled,
                         top_k, out_idx, scores, ws, ws_bytes, stream, &a);
}

// ------------------------------------------------------------------ sparse attention
size_t sparse_attn_workspace_bytes(int32_t n_q, int32_t n_heads, int32_t dv, int32_t top_k,
                                   int32_t q_dtype) {
  if (n_q < 1 || n_heads < 1 || dv < 1 || top_k < 1) return 0;
  return attn_plan(n_q, n_heads, dv, top_k, q_dtype).bytes;
}

enum AttnKind { ATTN_BF16, ATTN_FP8, ATTN_F32 };

// Checks the arguments of an attention call and fills the kernel arguments.
static ip_status attn_build(const char* fn, const ip_seqs* seqs, int32_t n_q, const int32_t* q_seq,
                            const int32_t* q_pos, const void* q, int32_t q_dtype, int32_t n_heads,
                            int32_t dk, int32_t dv, float scale, const ip_cache* k, const ip_cache* v,
                            const int32_t* sel_idx, int32_t top_k, void* out, float* lse, void* ws,
                            size_t ws_bytes, ip::AttnArgs& a, AttnKind& kind) {
  if (ip_status st = check_seqs(seqs, fn)) return st;
  if (ip_status st = check_cache(k, fn, "k")) return st;
  if (n_q < 1) return fail(IP_EINVAL, "%s: n_q must be >= 1", fn);
  if (!q || !sel_idx || !out) return fail(IP_EINVAL, "%s: q, sel_idx and out are required", fn);
  if (top_k < 1 || top_k > 2048) return fail(IP_EUNSUPPORTED, "%s: top_k must be in 1..2048 (got %d)", fn, top_k);
  if (!q_seq && n_q > seqs->batch) return fail(IP_EINVAL, "%s: q_seq is NULL but n_q > batch", fn);
  if (!(scale > 0.f)) return fail(IP_EINVAL, "%s: scale must be positive", fn);
  a = ip::AttnArgs{};
  a.L = layout_of(seqs);
  a.row0 = 0;
  a.n_rows = n_q;
  a.q_seq = q_seq;
  a.q_pos = q_pos;
  a.q = q;
  a.k = (const uint8_t*)k->data;
  a.k_stride = k->row_stride;
  a.sel = sel_idx;
  a.top_k = top_k;
  a.scale = scale;
  a.out = out;
  a.lse = lse;
  a.heads = n_heads;
  a.dk = dk;
  a.dv = dv;
  a.k_scale = nullptr;
  if (q_dtype == IP_BF16) {
    if ((k->dtype != IP_BF16 && k->dtype != IP_FP8_E4M3FN) || n_heads != ip::LAT_H || dk != ip::LAT_DK ||
        dv != ip::LAT_DV || k->row_dim < ip::LAT_DK)
      return fail(IP_EUNSUPPORTED, "%s: BF16 attention needs 64 heads, dk 576, dv 512 over a BF16 or FP8 latent cache", fn);
    if (v) return fail(IP_EUNSUPPORTED, "%s: BF16 latent attention takes V from the latent rows; pass v = NULL", fn);
    if (!seqs->page_table && (int64_t)seqs->batch * seqs->seq_stride > (int64_t(1) << 29))
      return fail(IP_EUNSUPPORTED, "%s: latent attention addresses token rows below 2^29 (batch * seq_stride too large)", fn);
    if (n_q > 65535) return fail(IP_EUNSUPPORTED, "%s: n_q > 65535", fn);
    const AttnPlan p = attn_plan(n_q, n_heads, dv, top_k, q_dtype);
    if (p.bytes > 0 && (!ws || ws_bytes < p.bytes))
      return fail(IP_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, p.bytes, ws ? ws_bytes : 0);
    if (((uintptr_t)ws & 15) != 0) return fail(IP_EINVAL, "%s: ws must be 16-byte aligned", fn);
    a.v = nullptr;
    a.v_stride = 0;
    // a contiguous cache whose rows all start below 4 GB - 1 KB from its base can be
    // read with 32-bit offsets (buffer loads)
    a.k_off32 = !seqs->page_table &&
                (int64_t)seqs->batch * seqs->seq_stride * k->row_stride <= (int64_t(1) << 32) - 4096;
    a.n_split = p.n_split;
    a.blocks_per_split = p.blocks_per_split;
    a.part_o = (uint16_t*)ws;
    a.part_ml = p.n_split > 1 ? (float*)(a.part_o + (size_t)n_q * p.n_split * n_heads * dv) : nullptr;
    if (k->dtype == IP_FP8_E4M3FN) {
      a.k_scale = k->scale;
      kind = ATTN_FP8;
    } else {
      kind = ATTN_BF16;
    }
    return IP_OK;
  }
  if (q_dtype == IP_F32) {
    if (ip_status st = check_cache(v, fn, "v")) return st;
    if (k->dtype != IP_F32 || v->dtype != IP_F32 || n_heads < 1 || n_heads > 16 || dk < 4 || dk > 128 ||
        dv < 1 || dv > 128 || dk % 4 || dv % 4 || k->row_dim < dk || v->row_dim < dv)
      return fail(IP_EUNSUPPORTED, "%s: F32 attention needs F32 k/v caches, n_heads <= 16, dk and dv <= 128 and multiples of 4", fn);
    a.v = (const uint8_t*)v->data;
    a.v_stride = v->row_stride;
    a.k_off32 = 0;
    a.n_split = 1;
    a.blocks_per_split = top_k;
    a.part_o = nullptr;
    a.part_ml = nullptr;
    kind = ATTN_F32;
    return IP_OK;
  }
  return fail(IP_EUNSUPPORTED, "%s: q must be BF16 or F32", fn);
}

static ip_status attn_launch(const char* fn, const ip::AttnArgs& a, AttnKind kind, hipStream_t stream) {
  switch (kind) {
    case ATTN_BF16: return device_status(ip::launch_attn_bf16(a, stream), fn);
    case ATTN_FP8: return device_status(ip::launch_attn_fp8(a, stream), fn);
    default: return device_status(ip::launch_attn_f32(a, stream), fn);
  }
}

static ip_status attn_common(const char* fn, const ip_seqs* seqs, int32_t n_q, const int32_t* q_seq,
                             const int32_t* q_pos, const void* q, int32_t q_dtype, int32_t n_heads,
                             int32_t dk, int32_t dv, float scale, const ip_cache* k, const ip_cache* v,
                             const int32_t* sel_idx, int32_t top_k, void* out, float* lse, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  ip::AttnArgs a;
  AttnKind kind;
  if (ip_status st = attn_build(fn, seqs, n_q, q_seq, q_pos, q, q_dtype, n_heads, dk, dv, scale, k, v, sel_idx,
                                top_k, out, lse, ws, ws_bytes, a, kind))
    return st;
  return attn_launch(fn, a, kind, stream);
}

ip_status sparse_attn_decode(const ip_seqs* seqs, const void* q, int32_t q_dtype, int32_t n_heads,
                             int32_t dk, int32_t dv, float scale, const ip_cache* k, const ip_cache* v,
                             const int32_t* sel_idx, int32_t top_k, void* out, float* lse, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  if (!seqs) return fail(IP_EINVAL, "sparse_attn_decode: seqs is NULL");
  return attn_common("sparse_attn_decode", seqs, seqs->batch, nullptr, nullptr, q, q_dtype, n_heads, dk, dv,
                     scale, k, v, sel_idx, top_k, out, lse, ws, ws_bytes, stream);
}

ip_status sparse_attn_prefill(const ip_seqs* seqs, int32_t n_q, const int32_t* q_seq, const int32_t* q_pos,
                              const void* q, int32_t q_dtype, int32_t n_heads, int32_t dk, int32_t dv,
                              float scale, const ip_cache* k, const ip_cache* v, const int32_t* sel_idx,
                              int32_t top_k, void* out, float* lse, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  if (!q_pos) return fail(IP_EINVAL, "sparse_attn_prefill: q_pos is required");
  return attn_common("sparse_attn_prefill", seqs, n_q, q_seq, q_pos, q, q_dtype, n_heads, dk, dv, scale, k, v,
                     sel_idx, top_k, out, lse, ws, ws_bytes, stream);
}

// ------------------------------------------------------------------ fused decode step
// workspace: the indexer's, the attention's, then per sequence a ready word, then the
// one-launch step's own per-wave lists (zero between calls)
struct StepPlan {
  ScorePlan score;
  AttnPlan attn;
  size_t idx_bytes, attn_bytes, ready_bytes, list_bytes, total;
};

static StepPlan step_plan(const ip_seqs* seqs, int32_t top_k, int32_t n_heads, int32_t dv, int32_t q_dtype,
                          bool scores_given) {
  StepPlan p;
  p.score = score_plan(seqs, seqs->batch, scores_given);
  p.attn = attn_plan(seqs->batch, n_heads, dv, top_k, q_dtype);
  p.idx_bytes = align256(p.score.total);
  p.attn_bytes = align256(p.attn.bytes);
  p.ready_bytes = align256((size_t)seqs->batch * 4);
  p.list_bytes = align256((size_t)seqs->batch * p.score.max_lists * (16 * 8 + 8));
  p.total = p.idx_bytes + p.attn_bytes + p.ready_bytes + p.list_bytes;
  return p;
}

extern "C" {

size_t indexpool_decode_step_workspace_bytes(const ip_seqs* seqs, int32_t top_k, int32_t n_heads, int32_t dv,
                                             int32_t q_dtype, int32_t scores_given) {
  if (!seqs || seqs->batch < 1 || top_k < 1 || n_heads < 1 || dv < 1 || seqs->max_seq_len < 1) return 0;
  return step_plan(seqs, top_k, n_heads, dv, q_dtype, scores_given != 0).total;
}

ip_status indexpool_decode_step(const ip_seqs* seqs, const void* kv_new, const ip_cache* kv, const void* v_new,
                                const ip_cache* v, const void* key_new, int32_t key_dtype, const ip_cache* keys,
                                const float* logit_new, float* logits, const ip_cache* pooled, const void* q_idx,
                                int32_t idx_dtype, int32_t idx_heads, int32_t idx_dim, const float* gates,
                                int32_t top_k, int32_t* out_idx, float* scores, const void* q, int32_t q_dtype,
                                int32_t n_heads, int32_t dk, int32_t dv, float scale, void* out, float* lse,
                                void* ws, size_t ws_bytes, hipStream_t stream) {
  const char* fn = "indexpool_decode_step";
  if (ip_status st = check_seqs(seqs, fn)) return st;
  if (!keys) return fail(IP_EINVAL, "%s: keys are required (the scoring reads the pooled keys)", fn);
  ip::AppendArgs app;
  if (ip_status st = build_append(fn, seqs, kv_new, kv, v_new, v, key_new, key_dtype, keys, logit_new, logits,
                                  pooled, app))
    return st;
  const int32_t B = seqs->batch;
  if (ip_status st = score_check(fn, seqs, B, nullptr, q_idx, idx_dtype, idx_heads, idx_dim, gates, pooled, top_k,
                                 out_idx))
    return st;
  if (n_heads < 1 || dv < 1) return fail(IP_EINVAL, "%s: n_heads and dv must be >= 1", fn);
  const StepPlan plan = step_plan(seqs, top_k, n_heads, dv, q_dtype, scores != nullptr);
  if (!ws || ws_bytes < plan.total)
    return fail(IP_EWORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, plan.total, ws ? ws_bytes : 0);
  if (((uintptr_t)ws & 255) != 0) return fail(IP_EINVAL, "%s: ws must be 256-byte aligned", fn);
  char* ws_idx = (char*)ws;
  char* ws_att = ws_idx + plan.idx_bytes;
  uint32_t* ready = (uint32_t*)(ws_att + plan.attn_bytes);
  char* step_lists = (char*)ready + plan.ready_bytes;
  ip::AttnArgs a;
  AttnKind kind;
  if (ip_status st = attn_build(fn, seqs, B, nullptr, nullptr, q, q_dtype, n_heads, dk, dv, scale, kv, v, out_idx,
                                top_k, out, lse, plan.attn_bytes ? ws_att : nullptr, plan.attn_bytes, a, kind))
    return st;
  // one launch when the selection is fused into the scoring (FP8 keys, every row in
  // one pass, rows short enough for the per-wave lists: the merge of one workgroup
  // of 4 waves is slower than the standalone scoring's 8-wave selection otherwise)
  // and the attention is the split bf16 latent kernel
  if (kind == ATTN_BF16 && pooled->dtype == IP_FP8_E4M3FN && plan.score.rows_per_pass >= B && plan.score.max_lists > 0 &&
      ((uintptr_t)kv_new & 15) == 0 && app.kv_row_bytes >= ip::LAT_DK * 2) {
    ip::StepArgs st;
    st.score = score_args(seqs, plan.score, 0, B, nullptr, nullptr, q_idx, idx_heads, idx_dim, gates, pooled, top_k,
                          out_idx, scores, ws_idx, &app);
    // the step's own lists (zero between calls: the combine clears them)
    st.score.lists = (uint64_t*)step_lists;
    st.score.lists_meta = (uint2*)(step_lists + (size_t)B * plan.score.max_lists * 16 * 8);
    st.score.step = 1;
    st.attn = a;
    st.attn.sel_ready = ready;
    st.attn.k_new = (const uint8_t*)kv_new;
    st.attn.k_new_stride = app.kv_row_bytes;
    st.attn.step_lists = st.score.lists;
    st.attn.step_meta = st.score.lists_meta;
    st.attn.step_max_lists = st.score.max_lists;
    st.attn.step_scores = st.score.scores;
    st.attn.step_ld = st.score.ld;
    st.attn.step_gm = st.score.gm;
    st.attn.step_gld = st.score.gld;
    st.attn.sel_out = out_idx;
    if (ip::decode_step_supported(st)) return device_status(ip::launch_decode_step(st, stream), fn);
  }
  // otherwise: the indexer call (with the append), then the attention
  if (ip_status st = score_topk_impl(fn, seqs, B, nullptr, nullptr, q_idx, idx_dtype, idx_heads, idx_dim, gates,
                                     pooled, top_k, out_idx, scores, ws_idx, plan.idx_bytes, stream, &app))
    return st;
  return attn_launch(fn, a, kind, stream);
}

}  // extern "C"

// ------------------------------------------------------------------ KDA decode step
ip_status kda_decode_step(int32_t batch, int32_t n_heads, int32_t head_dim, const void* xq, const void* xk,
                          const void* xv, int32_t x_dtype, const float* alpha, const float* beta,
                          const float* conv_w, const float* conv_in, float* conv_out, float* state, float* out,
                          hipStream_t stream) {
  const char* fn = "kda_decode_step";
  if (batch < 1 || batch > 65535 || n_heads < 1 || n_heads > 65535)
    return fail(IP_EINVAL, "%s: batch and n_heads must be in 1..65535 (got %d, %d)", fn, batch, n_heads);
  if (head_dim != ip::KDA_D) return fail(IP_EUNSUPPORTED, "%s: head_dim must be 128 (got %d)", fn, head_dim);
  if (x_dtype != IP_BF16) return fail(IP_EUNSUPPORTED, "%s: xq, xk, xv must be BF16", fn);
  if (!xq || !xk || !xv || !alpha || !beta || !conv_w || !conv_in || !conv_out || !state || !out)
    return fail(IP_EINVAL, "%s: every pointer is required", fn);
  const uintptr_t cb = (uintptr_t)batch * 9 * n_heads * ip::KDA_D * sizeof(float);
  const uintptr_t ci = (uintptr_t)conv_in, co = (uintptr_t)conv_out;
  if (ci < co + cb && co < ci + cb)
    return fail(IP_EINVAL, "%s: conv_in and conv_out must not overlap", fn);
  for (const void* p : {(const void*)conv_w, (const void*)state, (const void*)out})
    if ((reinterpret_cast<uintptr_t>(p) & 15) != 0)
      return fail(IP_EINVAL, "%s: conv_w, state and out must be 16-byte aligned", fn);
  ip::KdaArgs a;
  a.batch = batch;
  a.heads = n_heads;
  a.xq = (const uint16_t*)xq;
  a.xk = (const uint16_t*)xk;
  a.xv = (const uint16_t*)xv;
  a.alpha = alpha;
  a.beta = beta;
  a.conv_w = conv_w;
  a.conv_in = conv_in;
  a.conv_out = conv_out;
  a.state = state;
  a.out = out;
  return device_status(ip::launch_kda_decode(a, stream), fn);
}

ip_status kda_prefill_chunk(int32_t batch, int32_t n_tokens, int32_t n_heads, int32_t head_dim, const void* xq,
                            const void* xk, const void* xv, int32_t x_dtype, const float* alpha, const float* beta,
                            const float* conv_w, const float* conv_in, float* conv_out, float* state, float* out,
                            hipStream_t stream) {
  const char* fn = "kda_prefill_chunk";
  if (batch < 1 || batch > 65535 || n_heads < 1 || n_heads > 16383)
    return fail(IP_EINVAL, "%s: batch must be in 1..65535 and n_heads in 1..16383 (got %d, %d)", fn, batch, n_heads);
  if (n_tokens < 0) return fail(IP_EINVAL, "%s: n_tokens must be >= 0 (got %d)", fn, n_tokens);
  if (head_dim != ip::KDA_D) return fail(IP_EUNSUPPORTED, "%s: head_dim must be 128 (got %d)", fn, head_dim);
  if (x_dtype != IP_BF16) return fail(IP_EUNSUPPORTED, "%s: xq, xk, xv must be BF16", fn);
  if (!conv_w || !conv_in || !conv_out || !state || (n_tokens > 0 && (!xq || !xk || !xv || !alpha || !beta || !out)))
    return fail(IP_EINVAL, "%s: a required pointer is NULL", fn);
  const uintptr_t cb = (uintptr_t)batch * 9 * n_heads * ip::KDA_D * sizeof(float);
  const uintptr_t ci = (uintptr_t)conv_in, co = (uintptr_t)conv_out;
  if (ci < co + cb && co < ci + cb)
    return fail(IP_EINVAL, "%s: conv_in and conv_out must not overlap", fn);
  for (const void* p : {(const void*)conv_w, (const void*)state, xq, xk, xv, (const void*)alpha})
    if ((reinterpret_cast<uintptr_t>(p) & 15) != 0)
      return fail(IP_EINVAL, "%s: conv_w, state, xq, xk, xv and alpha must be 16-byte aligned", fn);
  ip::KdaChunkArgs a;
  a.batch = batch;
  a.heads = n_heads;
  a.n_tokens = n_tokens;
  a.xq = (const uint16_t*)xq;
  a.xk = (const uint16_t*)xk;
  a.xv = (const uint16_t*)xv;
  a.alpha = alpha;
  a.beta = beta;
  a.conv_w = conv_w;
  a.conv_in = conv_in;
  a.conv_out = conv_out;
  a.state = state;
  a.out = out;
  return device_status(ip::launch_kda_chunk(a, stream), fn);
}

// ------------------------------------------------------------------ no-allocation indexer
}  // extern "C"

namespace {

// Workspace of index_score_topk_noalloc: one copy per GPU the library runs on,
// held until the process ends.  Host code never passes the array's name to a
// kernel (on the host it is a stand-in, not a device address): it uses the address
// hipGetSymbolAddress returned for the device, kept in g_scratch_ptr.
constexpr size_t kScratchBytes = size_t(8) << 20;
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];         // per device: the array's device address, or null

__global__ void zero_words(uint4* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

// The current device's scratch address; on the first call for a device, the
// symbol address is looked up (with that device current) and the array is
// cleared on `stream` by a fill kernel (the per-row counters must start at zero;
// every call leaves them at zero again).
ip_status scratch_for_current_device(const char* fn, hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(IP_EDEVICE, "%s: no usable current device (%s)", fn, hipGetErrorString(e));
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr)
      return fail(IP_EDEVICE, "%s: hipGetSymbolAddress(scratch) failed: %s", fn, hipGetErrorString(e));
    hipLaunchKernelGGL(zero_words, dim3(256), dim3(256), 0, stream, (uint4*)ptr, kScratchBytes / 16);
    e = hipGetLastError();
    if (e != hipSuccess) return fail(IP_EDEVICE, "%s: clearing the scratch failed: %s", fn, hipGetErrorString(e));
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return IP_OK;
}

}  // namespace

extern "C" {

size_t index_score_topk_noalloc_max_bytes(void) { return kScratchBytes; }

ip_status index_score_topk_noalloc(const ip_seqs* seqs, int32_t n_q, const int32_t* q_seq,
                                   const int32_t* q_pos, const void* q_idx, int32_t q_dtype,
                                   int32_t n_heads, int32_t head_dim, const float* gates,
                                   const ip_cache* pooled, int32_t top_k, int32_t* out_idx,
                                   float* scores, hipStream_t stream) {
  const char* fn = "index_score_topk_noalloc";
  if (ip_status st = check_seqs(seqs, fn)) return st;
  if (n_q < 1 || top_k < 1) return fail(IP_EINVAL, "%s: n_q and top_k must be >= 1", fn);
  const size_t need = score_plan(seqs, n_q, scores != nullptr).total;
  if (need > kScratchBytes)
    return fail(IP_EWORKSPACE, "%s: this call needs %zu bytes of workspace, above the built-in %zu; call "
                "index_score_topk with a workspace instead", fn, need, kScratchBytes);
  void* ws = nullptr;
  if (ip_status st = scratch_for_current_device(fn, stream, &ws)) return st;
  return score_topk_impl(fn, seqs, n_q, q_seq, q_pos, q_idx, q_dtype, n_heads, head_dim, gates, pooled, top_k,
                         out_idx, scores, ws, kScratchBytes, stream, nullptr);
}

}  // extern "C"
