// Host metadata builder: validates a batch and turns it into work lists.
//
// «FlashAttention y FlashInfer», §Responsabilidades: the builder splits the
// batch into decodes and prefills, fills the per-sequence metadata and computes
// the kernel schedule ahead of time; the FlashInfer builder also reorders the
// batch so decodes come first (closing paragraph of §Flujo de datos).  Here the
// order is recorded (a stable partition) and the schedule walks it: decode work
// items first, then prefill work items.  Output rows keep the caller's order.
//
// «El especialista del plato estrella», §Qué aporta FlashInfer: with a shared
// prefix the prefix attention is scheduled once for all query rows and merged
// with each sequence's suffix attention through the LSE.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "internal.h"

namespace pa {

PrefillShape prefill_shape(int group, int tiles, int max_heads) {
  PrefillShape s{};
  s.tiles = tiles;
  int hpw = 1;
  for (int c : {8, 4, 2}) {
    if (c <= max_heads && group % c == 0) {
      hpw = c;
      break;
    }
  }
  s.heads_per_wg = hpw;
  s.tiles_per_head = tiles / hpw;
  s.rows_per_item = 16 * s.tiles_per_head;
  s.head_groups = group / hpw;
  return s;
}

namespace {

constexpr int kPrefixChunk = 1024;  // shared-prefix keys per cascade work item (prefix before the decode)

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// Share of the resident decode wave groups that the decode lists take when
// prefills run beside them: the decode's time alone over the sum of both
// parts' times alone, estimated from the KV bytes the decodes read (at the
// decode kernel's rate, about 6 TB/s) and the attention FLOPs of the side
// stream (the prefills', and a shared-prefix pass's: every decode row against
// the prefix; at the prefill kernel's rate: about 0.9 PFLOP/s on bf16 MFMA,
// 0.7 over an e4m3 pool, whose prefill widens the codes on the way to LDS,
// far less in fp32), kept within [0.25, 0.75].  On MI355X the decode keeps HBM near its
// rate with about 70 % of the groups, while the prefill waits for free CUs
// when the decode holds them all: on a mixed step of 192 decodes and four
// 512-token chunks the step takes 1.29 ms at 70-75 % against 1.41 ms at 100 %;
// over an e4m3 pool 0.78 ms at 60 % (the share the 0.7 rate gives) against
// 0.79-0.80 ms at 50-55 % and 0.81 ms at 65.5 % (the share of the 0.9 rate).
double decode_share(const pa_params& p, int B, const int32_t* qsl, const int32_t* seq_lens, int64_t dec_tokens,
                    int32_t n_decode_rows) {
  constexpr double kDecodeBytesPerSec = 6.0e12;
  const double pre_flops_per_sec = p.dtype != PA_BF16                ? 0.1e15
                                   : p.kv_dtype == PA_KV_FP8_E4M3 ? 0.7e15
                                                                  : 0.9e15;
  const double elem = p.kv_dtype == PA_KV_FP8_E4M3 ? 1.0 : (p.dtype == PA_BF16 ? 2.0 : 4.0);
  double pairs = 0.0;  // (query row, visible key) pairs of the prefills, per query head
  for (int b = 0; b < B; ++b) {
    const double qb = qsl[b + 1] - qsl[b];
    if (qb <= 1) continue;
    const double L = seq_lens[b];
    pairs += p.causal ? qb * (L - qb) + 0.5 * qb * (qb + 1.0) : qb * L;
  }
  // the shared-prefix pass runs on the same side stream: every decode row
  // against the P prefix keys
  pairs += (double)n_decode_rows * p.common_prefix_len;
  const double t_dec = (double)dec_tokens * 2.0 * p.num_kv_heads * p.head_size * elem / kDecodeBytesPerSec;
  const double t_pre = 4.0 * p.head_size * p.num_heads * pairs / pre_flops_per_sec;
  if (t_dec + t_pre <= 0.0) return 0.75;
  return std::min(0.75, std::max(0.25, t_dec / (t_dec + t_pre)));
}

// Rates of this library's kernels on one MI355X CU (measured on a shared-prefix
// batch): the 8-wave wide prefill executes about 3.6 TFLOP/s of MFMA work per
// CU on long non-causal units, and a decode workgroup draws about 25 GB/s
// from HBM (the decode as a whole at most about 6.5 TB/s).  A unit's fixed
// cost (its Q rows in, the first K/V block's latency, its output out) is
// worth about 192 keys.
// A decode work item's start (its row of Q, its first block-table entries,
// then its first K/V step, one after the other) costs a decode workgroup
// time; the balanced lists count it in keys.  Timing every list of the
// decode-only batch (256 lists, one per CU) and fitting their end times to
// keys, items and XCD gives 0.112 us per key and 1.4 us per item (16 keys'
// worth) for decodes alone, and 2.3-2.5 us (about 24 keys) for the suffix
// lists beside a shared-prefix pass in the same launch; beside prefills a
// count of 64 keys still times best.
constexpr int kDecodeItemKeysAlone = 16;
constexpr int kDecodeItemKeysBesidePrefix = 24;
constexpr int kDecodeItemKeys = 64;
// The same fit shows the lists on even-numbered XCDs (workgroup index even:
// workgroups are dealt to the eight XCDs in turn) ending about 1.6 % later
// than those on odd ones for equal work, on every MI355X timed; lists of
// decodes alone are sized W - W/128 on even and W + W/128 on odd XCDs.
inline int xcd_list_budget(int W, int64_t workgroup) { return workgroup % 2 == 0 ? W - W / 128 : W + W / 128; }
constexpr double kPrefixFlopsPerCu = 3.6e12;
constexpr double kDecodeBytesPerCu = 25.0e9;
constexpr double kDecodeBytesAll = 6.5e12;
constexpr int kUnitOverheadKeys = 192;

pa_status fail(std::string& err, pa_status st, const char* fmt, long long a = 0, long long b = 0,
               long long c = 0) {
  char buf[256];
  std::snprintf(buf, sizeof(buf), fmt, a, b, c);
  err = buf;
  return st;
}

}  // namespace

pa_status build_host_plan(const pa_params& p, const int32_t* qsl, const int32_t* seq_lens,
                          const int32_t* block_table, int num_cus, int decode_wgs_per_cu, HostPlan& hp,
                          std::string& err) {
  // ---- validation («FlashAttention y FlashInfer», §Límites y fallos;
  //      «AttentionBackend: capa de abstracción», §Límites y fallos)
  const int B = p.num_seqs;
  if (B < 0) return fail(err, PA_ERR_INVALID_ARG, "num_seqs %lld < 0", B);
  if (!qsl || !seq_lens) return fail(err, PA_ERR_INVALID_ARG, "query_start_loc / seq_lens is NULL");
  if (p.num_heads < 1 || p.num_kv_heads < 1)
    return fail(err, PA_ERR_INVALID_ARG, "num_heads %lld / num_kv_heads %lld must be >= 1", p.num_heads,
                p.num_kv_heads);
  if (p.num_heads % p.num_kv_heads != 0)
    return fail(err, PA_ERR_INVALID_ARG, "num_heads %lld is not a multiple of num_kv_heads %lld",
                p.num_heads, p.num_kv_heads);
  if (p.block_size < 16 || p.block_size % 16 != 0)
    return fail(err, PA_ERR_INVALID_ARG, "block_size %lld must be a positive multiple of 16", p.block_size);
  if (p.head_size != 64 && p.head_size != 128)
    return fail(err, PA_ERR_UNSUPPORTED, "head_size %lld not built (64, 128)", p.head_size);
  if (p.dtype != PA_BF16 && p.dtype != PA_FP32)
    return fail(err, PA_ERR_UNSUPPORTED, "dtype %lld not built (PA_BF16, PA_FP32)", p.dtype);
  if (p.kv_dtype != PA_KV_SAME && p.kv_dtype != PA_KV_FP8_E4M3)
    return fail(err, PA_ERR_INVALID_ARG, "kv_dtype %lld (PA_KV_SAME, PA_KV_FP8_E4M3)", p.kv_dtype);
  if (p.kv_dtype == PA_KV_FP8_E4M3 && p.dtype != PA_BF16)
    return fail(err, PA_ERR_UNSUPPORTED, "an e4m3 pool is built for bf16 queries only");
  if (p.kv_layout != PA_KV_NHD && p.kv_layout != PA_KV_HND)
    return fail(err, PA_ERR_INVALID_ARG, "kv_layout %lld (PA_KV_NHD, PA_KV_HND)", p.kv_layout);
  if ((int64_t)p.block_size * p.head_size > INT32_MAX / 2 || (int64_t)p.num_kv_heads * p.head_size > INT32_MAX / 2)
    return fail(err, PA_ERR_INVALID_ARG, "block_size * head_size or num_kv_heads * head_size too large");
  if (p.num_blocks < 1) return fail(err, PA_ERR_INVALID_ARG, "num_blocks %lld < 1", p.num_blocks);
  if (p.max_blocks_per_seq < 1)
    return fail(err, PA_ERR_INVALID_ARG, "max_blocks_per_seq %lld < 1", p.max_blocks_per_seq);
  if (p.causal != 0 && p.causal != 1) return fail(err, PA_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (p.check_metadata != 0 && p.check_metadata != 1)
    return fail(err, PA_ERR_INVALID_ARG, "check_metadata must be 0 or 1");
  if (!std::isfinite(p.scale) || !(p.scale > 0.f))
    return fail(err, PA_ERR_INVALID_ARG, "scale must be positive and finite");
  if (p.kv_split_tokens < 0 || p.kv_split_tokens % 32 != 0)
    return fail(err, PA_ERR_INVALID_ARG, "kv_split_tokens %lld must be 0 or a positive multiple of 32",
                p.kv_split_tokens);
  if (p.common_prefix_len < 0) return fail(err, PA_ERR_INVALID_ARG, "common_prefix_len < 0");
  if (qsl[0] != 0) return fail(err, PA_ERR_INVALID_ARG, "query_start_loc[0] = %lld, must be 0", qsl[0]);

  const int bs = p.block_size;
  const int mb = p.max_blocks_per_seq;
  for (int b = 0; b < B; ++b) {
    const int64_t qb = (int64_t)qsl[b + 1] - qsl[b];
    if (qb < 1)
      return fail(err, PA_ERR_INVALID_ARG, "sequence %lld has %lld query tokens (need >= 1)", b, qb);
    if (seq_lens[b] < qb)
      return fail(err, PA_ERR_INVALID_ARG, "sequence %lld: seq_len %lld < query tokens %lld", b,
                  seq_lens[b], qb);
    if (ceil_div(seq_lens[b], bs) > mb)
      return fail(err, PA_ERR_INVALID_ARG, "sequence %lld needs %lld blocks > max_blocks_per_seq %lld", b,
                  ceil_div(seq_lens[b], bs), mb);
    if (block_table) {
      const int nb = (int)ceil_div(seq_lens[b], bs);
      for (int j = 0; j < nb; ++j) {
        const int32_t id = block_table[(int64_t)b * mb + j];
        if (id < 0 || id >= p.num_blocks)
          return fail(err, PA_ERR_INVALID_ARG, "block_table[%lld][%lld] = %lld outside the pool", b, j, id);
      }
    }
  }
  if (B > 0 && (int64_t)qsl[B] > INT32_MAX / 2)
    return fail(err, PA_ERR_INVALID_ARG, "too many tokens");

  const int P = p.common_prefix_len;
  if (P > 0) {
    if (!block_table) return fail(err, PA_ERR_INVALID_ARG, "cascade (common_prefix_len > 0) needs block_table");
    if (P % bs != 0)
      return fail(err, PA_ERR_INVALID_ARG, "common_prefix_len %lld is not a multiple of block_size %lld", P, bs);
    for (int b = 0; b < B; ++b) {
      const int ctx = seq_lens[b] - (qsl[b + 1] - qsl[b]);
      if (ctx < P)
        return fail(err, PA_ERR_INVALID_ARG, "common_prefix_len %lld exceeds the context %lld of sequence %lld",
                    P, ctx, b);
      for (int j = 0; j < P / bs; ++j)
        if (block_table[(int64_t)b * mb + j] != block_table[j])
          return fail(err, PA_ERR_INVALID_ARG, "prefix block %lld of sequence %lld differs from sequence 0", j, b);
    }
  }

  // ---- metadata: decode / prefill split, decode-first stable order
  hp = HostPlan{};
  hp.p = p;
  const int H = p.num_heads, Hkv = p.num_kv_heads, g = H / Hkv;
  hp.T = B > 0 ? qsl[B] : 0;
  hp.qsl.assign(qsl, qsl + B + 1);
  hp.seq_lens.assign(seq_lens, seq_lens + B);
  if (block_table) hp.block_table.assign(block_table, block_table + (int64_t)B * mb);
  hp.order.reserve(B);
  hp.is_decode.resize(B);
  int nd = 0, ndt = 0, np = 0, npt = 0;
  for (int b = 0; b < B; ++b) {
    const int qb = qsl[b + 1] - qsl[b];
    hp.is_decode[b] = qb == 1;
    if (qb == 1) {
      hp.order.push_back(b);
      ++nd;
      ndt += 1;
    }
  }
  for (int b = 0; b < B; ++b) {
    const int qb = qsl[b + 1] - qsl[b];
    if (qb != 1) {
      hp.order.push_back(b);
      ++np;
      npt += qb;
    }
  }
  if (P > 0) hp.prefix_blocks.assign(block_table, block_table + P / bs);

  // ---- schedule
  int64_t dec_tokens = 0;
  for (int i = 0; i < nd; ++i) dec_tokens += seq_lens[hp.order[i]] - P;
  const int dec_units = Hkv * ((g + 15) / 16);
  const int dec_nw = decode_waves_per_wg(dec_units);
  const bool balanced = p.kv_split_tokens == 0 && nd > 0 && decode_wgs_per_cu > 0;
  // the wide kernel needs both tiles of a wave on one head (at most tiles / 2 heads)
  if (use_wide_prefill(p.dtype, p.head_size, p.kv_dtype)) {
    const int tiles = wide_prefill_tiles(nd > 0 && np > 0, p.kv_dtype);
    hp.ps = prefill_shape(g, tiles, tiles / 2);
  } else {
    hp.ps = prefill_shape(g, 8, 8);
  }
  int n_pc = P > 0 ? (int)ceil_div(P, kPrefixChunk) : 0;

  // Shared prefix beside the decode.  With decodes only (bf16 pool, head size
  // 128, automatic split, 8-wave decode workgroups) the prefix pass runs at
  // the same time as the decode, in the same launch, on CUs of its own: one
  // 8-wave workgroup per prefix unit (chunk, column group, KV head), each
  // filling a CU's registers, while the decode lists are sized for the
  // remaining CUs.  The chunk count sets how many CUs the prefix
  // takes; it is chosen so that the two finish together (the rates above).
  if (P > 0 && np == 0 && balanced && use_wide_prefill(p.dtype, p.head_size, p.kv_dtype) &&
      p.kv_dtype == PA_KV_SAME && dec_nw == 8) {
    const PrefillShape s16 = prefill_shape(g, 16, 8);
    const int per_chunk = (int)ceil_div(hp.T, s16.rows_per_item) * Hkv * s16.head_groups;
    const double dec_bytes = (double)dec_tokens * 2.0 * Hkv * p.head_size * 2.0;
    double best_t = 0.0;
    int best_c = 0;
    for (int c = 1; c <= ceil_div(P, 64) && (int64_t)c * per_chunk <= num_cus - 8; ++c) {
      const int len = (int)round_up(ceil_div(P, c), 64);
      const int units = (int)ceil_div(P, len) * per_chunk;
      const double t_pfx = 16.0 * s16.tiles * (len + kUnitOverheadKeys) * 4.0 * p.head_size / kPrefixFlopsPerCu;
      const double t_dec = dec_bytes / std::min(kDecodeBytesAll, (num_cus - units) * kDecodeBytesPerCu);
      const double t = std::max(t_pfx, t_dec);
      if (best_c == 0 || t < best_t) {
        best_t = t;
        best_c = c;
      }
    }
    if (best_c > 0) {
      hp.ps = s16;
      n_pc = best_c;
      hp.prefix_beside = true;
    }
  }
  const int QB = hp.ps.rows_per_item;
  const int pc_len = P > 0 ? (int)round_up(ceil_div(P, n_pc), 64) : 0;
  if (P > 0) n_pc = (int)ceil_div(P, pc_len);  // no empty chunk

  // Decode schedule.  With the automatic split the decodes get balanced work
  // lists: the decode keys (past the shared prefix, if any), sequence after
  // sequence, are cut into equal lists, one per group of waves resident at
  // once, so all of them finish together (a list may end one sequence and
  // start the next; each piece is an item with its own partial record).
  // Beside prefills the lists take only a share of the resident groups (see
  // decode_share) and the prefill runs on the rest of the machine meanwhile;
  // beside a shared-prefix pass (above) they cover the CUs it leaves free,
  // and otherwise a shared-prefix pass runs before the decode.
  // With an explicit split each decode is cut into equal parts of at most
  // `split` keys, one item per list, longest first.
  int split = p.kv_split_tokens;
  int list_tokens = 0;
  // decodes alone: the start cost of an item and the XCD budgets measured for
  // them (see kDecodeItemKeysAlone); otherwise the figure that times best
  // beside other work, and one budget for every list
  const bool decodes_alone = np == 0 && P == 0;
  const int item_keys = decodes_alone       ? kDecodeItemKeysAlone
                        : hp.prefix_beside ? kDecodeItemKeysBesidePrefix
                                           : kDecodeItemKeys;
  // list i is workgroup i; the whole chip (256 CUs, eight XCDs), where the
  // XCD timings were taken
  const bool xcd_budgets = decodes_alone && dec_units == dec_nw && num_cus == 256;
  auto list_budget = [&](int W, int64_t list) { return xcd_budgets ? xcd_list_budget(W, list) : W; };
  if (balanced) {
    // resident list groups: workgroups per CU x CUs / workgroups per list
    const int prefix_cus = hp.prefix_beside ? n_pc * (int)ceil_div(hp.T, QB) * Hkv * hp.ps.head_groups : 0;
    const int dec_cus = std::max(num_cus - prefix_cus, 1);
    int64_t lanes = std::max<int64_t>(1, (int64_t)decode_wgs_per_cu * dec_cus * dec_nw / dec_units);
    if (np > 0)
      lanes = std::max<int64_t>(1, (int64_t)(lanes * decode_share(p, B, qsl, seq_lens, dec_tokens, nd)));
    const int64_t n_lists = std::max<int64_t>(1, std::min<int64_t>(lanes, ceil_div(dec_tokens, 256)));
    // Each list gets a budget of keys (W, or W -+ W/128 by XCD for decodes
    // alone when each list is one workgroup), each of its items counting
    // item_keys more.  A list is closed with up to 31 (after an item) or
    // 31 + item_keys (before one) of its budget unused, so W is the smallest
    // budget from the even share up whose cut needs at most n_lists lists:
    // keys never spill into a second, nearly empty round of workgroups, and
    // (the budget moving in steps of one key) no resident group is left
    // without a list by a budget rounded up.
    auto lists_needed = [&](int W) {
      int64_t n = 0;
      int filled = 0;
      for (int oi = 0; oi < nd; ++oi) {
        const int L = seq_lens[hp.order[oi]];
        for (int k0 = P; k0 < L;) {
          if (list_budget(W, n) - filled - item_keys < 32) {
            ++n;
            filled = 0;
          }
          filled += item_keys;
          const int room = list_budget(W, n) - filled;
          const int take = L - k0 <= room ? L - k0 : room / 32 * 32;
          k0 += take;
          filled += take;
          if (list_budget(W, n) - filled < 32) {
            ++n;
            filled = 0;
          }
        }
      }
      return n + (filled > 0 ? 1 : 0);
    };
    // (every sequence is at least one item: the even share of keys and item
    // starts is a lower bound)
    int W = (int)std::max<int64_t>(64 + item_keys, ceil_div(dec_tokens + (int64_t)nd * item_keys, n_lists));
    while (lists_needed(W) > n_lists) W += 32;
    // back from the first fitting step of 32 to the smallest fitting budget
    const int W32 = W;
    for (int lower = W32 - 1; lower > W32 - 32 && lower >= 64 + item_keys && lists_needed(lower) <= n_lists; --lower)
      W = lower;
    list_tokens = W;
    split = list_tokens;
  } else if (split == 0) {
    const int64_t target_items = std::max<int64_t>(1, (int64_t)32 * std::max(num_cus, 1) / Hkv);
    split = (int)std::min<int64_t>(8192, std::max<int64_t>(256, round_up(ceil_div(dec_tokens, target_items), 32)));
  }

  std::vector<int32_t> contrib(hp.T, 0);
  int64_t dec_read = 0, pre_read = 0, pfx_read = 0;
  if (balanced) {
    // Cuts inside a sequence fall on multiples of 32 keys (the decode kernel's
    // 16-key tiles must not straddle a physical block); a list is closed once
    // less than 32 keys of room are left, or before an item that would start
    // with less (the same cut lists_needed counts).
    int filled = 0;  // budget used in the open list
    hp.decode_lists.push_back(0);
    for (int oi = 0; oi < nd; ++oi) {
      const int b = hp.order[oi];
      const int L = seq_lens[b];
      int part = 0;
      for (int k0 = P; k0 < L;) {
        if (list_budget(list_tokens, (int64_t)hp.decode_lists.size() - 1) - filled - item_keys < 32) {
          hp.decode_lists.push_back((int32_t)hp.decode_items.size());
          filled = 0;
        }
        const int Wl = list_budget(list_tokens, (int64_t)hp.decode_lists.size() - 1);
        filled += item_keys;
        const int room = Wl - filled;  // >= 32
        const int take = L - k0 <= room ? L - k0 : room / 32 * 32;
        WorkItem it{};
        it.seq = b;
        it.row0 = qsl[b];
        it.nrows = 1;
        it.lim0 = L - 1;
        it.kv_begin = k0;
        it.kv_end = k0 + take;
        it.slot = n_pc + part++;
        it.causal = 0;
        hp.decode_items.push_back(it);
        dec_read += take;
        k0 += take;
        filled += take;
        if (Wl - filled < 32) {
          hp.decode_lists.push_back((int32_t)hp.decode_items.size());
          filled = 0;
        }
      }
      contrib[qsl[b]] = n_pc + part;
    }
    if (filled > 0) hp.decode_lists.push_back((int32_t)hp.decode_items.size());
  }
  for (int oi = 0; oi < B; ++oi) {
    const int b = hp.order[oi];
    const int qb = qsl[b + 1] - qsl[b];
    const int L = seq_lens[b];
    const int ctx = L - qb;
    if (qb == 1) {
      if (balanced) continue;
      const int span = L - P;
      const int n = (int)ceil_div(span, split);
      const int part = (int)round_up(ceil_div(span, n), 32);
      // n parts of equal size (multiple of 32, at most `split`): since
      // (n - 1) * part <= (n - 1) * split < span, every part is non-empty.
      for (int j = 0; j < n; ++j) {
        WorkItem it{};
        it.seq = b;
        it.row0 = qsl[b];
        it.nrows = 1;
        it.lim0 = L - 1;
        it.kv_begin = P + j * part;
        it.kv_end = std::min(L, P + (j + 1) * part);
        it.slot = n_pc + j;
        it.causal = 0;
        hp.decode_items.push_back(it);
        dec_read += it.kv_end - it.kv_begin;
      }
      contrib[qsl[b]] = n_pc + n;
    } else {
      for (int i0 = 0; i0 < qb; i0 += QB) {
        WorkItem it{};
        it.seq = b;
        it.row0 = qsl[b] + i0;
        it.nrows = std::min(QB, qb - i0);
        it.lim0 = ctx + i0;
        // prefill rows attend to their whole context in their own items, the
        // shared prefix included: many queries per key, so sharing the
        // prefix's reads would save little and cost partial records
        it.kv_begin = 0;
        it.kv_end = p.causal ? std::min(L, ctx + i0 + it.nrows) : L;
        it.slot = 0;
        it.causal = p.causal;
        hp.prefill_items.push_back(it);
        pre_read += (int64_t)(it.kv_end - it.kv_begin) * hp.ps.head_groups;
      }
      for (int r = qsl[b]; r < qsl[b + 1]; ++r) contrib[r] = 1;
    }
  }
  if (P > 0) {
    // The prefix pass covers the decode rows, run by run of consecutive rows
    // (one run in a decode-first batch).  Chunk-major: the row groups that
    // read one prefix chunk are dispatched back to back (on the same XCD), so
    // the chunk is fetched once into L2.
    std::vector<std::pair<int, int>> runs;  // decode rows [first, end)
    for (int b = 0; b < B; ++b) {
      if (qsl[b + 1] - qsl[b] != 1) continue;
      if (!runs.empty() && runs.back().second == qsl[b])
        runs.back().second += 1;
      else
        runs.push_back({qsl[b], qsl[b] + 1});
    }
    for (int j = 0; j < n_pc; ++j) {
      for (const auto& run : runs) {
        for (int r0 = run.first; r0 < run.second; r0 += QB) {
          WorkItem it{};
          it.seq = 0;
          it.row0 = r0;
          it.nrows = std::min(QB, run.second - r0);
          it.lim0 = 0;
          it.kv_begin = j * pc_len;
          it.kv_end = std::min(P, (j + 1) * pc_len);
          it.slot = j;
          it.causal = 0;
          if (it.kv_begin >= it.kv_end) continue;
          hp.prefix_items.push_back(it);
          pfx_read += (int64_t)(it.kv_end - it.kv_begin) * hp.ps.head_groups;
        }
      }
    }
  }
  // longest work first, so the tail of each launch is short items
  auto span = [](const WorkItem& a) { return (int64_t)(a.kv_end - a.kv_begin); };
  if (!balanced) {
    std::stable_sort(hp.decode_items.begin(), hp.decode_items.end(),
                     [&](const WorkItem& a, const WorkItem& b) { return span(a) > span(b); });
    hp.decode_lists.resize(hp.decode_items.size() + 1);
    for (size_t i = 0; i < hp.decode_lists.size(); ++i) hp.decode_lists[i] = (int32_t)i;
  }
  // prefill: sequences by their longest item, then each sequence's items
  // longest first; the workgroups in flight on one XCD then share the pages
  // of one or two sequences instead of the heads of many
  {
    std::vector<int64_t> seq_span(B, 0);
    for (const WorkItem& it : hp.prefill_items) seq_span[it.seq] = std::max(seq_span[it.seq], span(it));
    std::stable_sort(hp.prefill_items.begin(), hp.prefill_items.end(), [&](const WorkItem& a, const WorkItem& b) {
      if (seq_span[a.seq] != seq_span[b.seq]) return seq_span[a.seq] > seq_span[b.seq];
      if (a.seq != b.seq) return a.seq < b.seq;
      return span(a) > span(b);
    });
  }

  // the kernels read keys in 16-key tiles that must lie in one physical block
  for (const auto* v : {&hp.decode_items, &hp.prefill_items, &hp.prefix_items})
    for (const WorkItem& it : *v)
      if (it.kv_begin % 16 != 0 || it.kv_end <= it.kv_begin)
        return fail(err, PA_ERR_INVALID_ARG, "internal: work item keys [%lld, %lld) not 16-aligned or empty",
                    it.kv_begin, it.kv_end);

  // partial records: one range per row that merges several contributions
  hp.row_pbase.assign(hp.T, -1);
  hp.row_partials.assign(hp.T, 0);
  int next = 0;
  for (int r = 0; r < hp.T; ++r) {
    if (contrib[r] > 1) {
      hp.row_pbase[r] = next;
      hp.row_partials[r] = contrib[r];
      hp.merges.push_back(MergeRow{r, next, contrib[r], 0});
      next += contrib[r];
    }
  }
  hp.num_partials = next;

  pa_plan_info& in = hp.info;
  in.num_seqs = B;
  in.num_tokens = hp.T;
  in.num_decodes = nd;
  in.num_decode_tokens = ndt;
  in.num_prefills = np;
  in.num_prefill_tokens = npt;
  in.common_prefix_len = P;
  in.num_prefix_blocks = P / bs;
  in.num_decode_items = (int32_t)hp.decode_items.size();
  in.num_prefill_items = (int32_t)hp.prefill_items.size();
  in.num_prefix_items = (int32_t)hp.prefix_items.size();
  in.num_merge_rows = (int32_t)hp.merges.size();
  in.num_partials = hp.num_partials;
  in.kv_split_tokens = split;
  in.prefill_rows_per_item = hp.ps.rows_per_item;
  in.prefill_head_groups = hp.ps.head_groups;
  in.num_decode_lists = hp.decode_lists.empty() ? 0 : (int32_t)hp.decode_lists.size() - 1;
  in.decode_list_tokens = list_tokens;
  in.decode_tokens_read = dec_read * Hkv;
  in.prefill_tokens_read = pre_read * Hkv;
  in.prefix_tokens_read = pfx_read * Hkv;
  in.prefix_tokens_unique = (int64_t)P * Hkv;
  in.prefix_beside_decode = hp.prefix_beside ? 1 : 0;
  in.decode_item_keys = list_tokens > 0 ? item_keys : 0;
  in.decode_list_xcd_budgets = list_tokens > 0 && xcd_budgets ? 1 : 0;
  in.kv_tokens_read = in.decode_tokens_read + in.prefill_tokens_read + in.prefix_tokens_read;
  return PA_OK;
}

}  // namespace pa
