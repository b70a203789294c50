// Host check of the token-level top-k count and position arithmetic
// (block_sparse_attention_12_amd/csrc/tok_positions.h, the functions the
// token kernels call). Test infrastructure: built with g++ by
// tests/test_token_positions_cpu.py, with the undefined-behaviour sanitizer.
//
// A host model runs the kernels' chain for one (sequence, KV head) unit: the
// radix passes over 8-bit digits of the 32-bit keys (most significant first),
// the early stop once the boundary bin holds exactly the keys still to take,
// per-chunk counts of surely-taken and equal keys, and the ascending
// compaction (chunks of 4096 tokens, 16 consecutive tokens per thread, an
// exclusive prefix over threads). It checks
//   1. consistent inputs: the row equals the brute-force top-k (keys
//      descending, ties to the lower token) plus the kept initial and local
//      tokens, ascending;
//   2. inconsistent inputs (random histograms, chunk counts and stored words,
//      as a fault in another workgroup could leave them): every slot written
//      lies in [0, idx_cap), the count lies in [0, idx_cap], and no signed
//      arithmetic overflows (the sanitizer aborts on any).
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <algorithm>
#include <random>
#include <vector>

#include "../../block_sparse_attention_12_amd/csrc/tok_positions.h"

using namespace sa;

static const int kChunk = 4096, kPer = 16, kThreads = kChunk / kPer;

struct Windows {
    int64_t L, init_hi, local_lo, n_cand;
    bool choose, take_all;
};
static Windows windows(int64_t L, int top_k, int n_init, int n_local) {
    Windows w;
    w.L = L;
    w.init_hi = n_init < L ? n_init : L;
    const int64_t lo = L - n_local;
    w.local_lo = lo > w.init_hi ? lo : w.init_hi;
    w.n_cand = w.local_lo - w.init_hi;
    w.take_all = top_k >= w.n_cand;
    w.choose = !w.take_all && top_k > 0;
    return w;
}

// prefix / mask / remaining after `passes` passes over the given histograms
static void prefix_of(const std::vector<uint32_t> &hist, int passes, int top_k, uint32_t &prefix,
                      uint32_t &mask, int &remaining, bool &whole) {
    prefix = 0;
    mask = 0;
    remaining = top_k;
    whole = false;
    for (int p = 0; p < passes; ++p) {
        const TokDigit d = tok_digit_seq(&hist[p * 256], remaining);
        const int shift = 24 - 8 * p;
        prefix |= d.digit << shift;
        mask |= 255u << shift;
        remaining = tok_remaining_after(remaining, d.above);
        if (d.bcnt == (uint32_t)remaining) {
            whole = true;
            break;
        }
    }
}

struct Result {
    std::vector<int32_t> row;
    int cnt;
    int64_t bad_writes;
};

// The compaction of tok_write_kernel for every chunk, given the per-chunk
// counts and the stored (thr, take_eq word, mask).
static Result write_row(const std::vector<uint32_t> &keys, const Windows &w, bool whole_unused,
                        const std::vector<int32_t> &counts, uint32_t thr, uint32_t take_word,
                        uint32_t mask, int idx_cap) {
    (void)whole_unused;
    Result r;
    r.row.assign(idx_cap, -7);
    r.bad_writes = 0;
    const int take_eq = w.choose ? tok_take_eq(take_word) : 0;
    const int n_used = (int)((w.L + kChunk - 1) / kChunk);
    auto sums = [&](int upto, int64_t &sure, int64_t &eq) {
        sure = eq = 0;
        for (int c = 0; c < upto; ++c) {
            sure += counts[2 * c];
            eq += counts[2 * c + 1];
        }
    };
    int64_t sure, eq;
    sums(n_used, sure, eq);
    r.cnt = tok_row_total(sure, eq, take_eq, idx_cap);
    if (r.cnt < 0 || r.cnt > idx_cap) r.bad_writes++;
    for (int i = r.cnt; i < idx_cap; ++i) r.row[i] = -1;
    for (int chunk = 0; chunk < n_used; ++chunk) {
        const int64_t t0 = (int64_t)chunk * kChunk;
        int64_t sure_before, eq_before;
        sums(chunk, sure_before, eq_before);
        auto cand = [&](int64_t t) { return t >= w.init_hi && t < w.local_lo; };
        // per-thread equal-key counts and their exclusive prefix
        std::vector<int> n_eq(kThreads, 0), n_in(kThreads, 0);
        for (int th = 0; th < kThreads; ++th)
            for (int i = 0; i < kPer; ++i) {
                const int64_t t = t0 + th * kPer + i;
                if (w.choose && t < w.L && cand(t) && (keys[t] & mask) == thr) n_eq[th]++;
            }
        int64_t eq_scan = 0;
        std::vector<std::vector<bool>> in(kThreads, std::vector<bool>(kPer, false));
        for (int th = 0; th < kThreads; ++th) {
            int64_t eq_rank = eq_before + eq_scan;
            eq_scan += n_eq[th];
            for (int i = 0; i < kPer; ++i) {
                const int64_t t = t0 + th * kPer + i;
                bool x;
                if (t >= w.L) x = false;
                else if (!cand(t)) x = true;
                else if (w.take_all) x = true;
                else if (!w.choose) x = false;
                else if ((keys[t] & mask) > thr) x = true;
                else if ((keys[t] & mask) == thr) x = eq_rank++ < take_eq;
                else x = false;
                in[th][i] = x;
                n_in[th] += x ? 1 : 0;
            }
        }
        int scan = 0;
        for (int th = 0; th < kThreads; ++th) {
            int64_t pos = tok_first_pos(sure_before, eq_before, take_eq, scan);
            scan += n_in[th];
            for (int i = 0; i < kPer; ++i)
                if (in[th][i]) {
                    if (tok_slot_ok(pos, idx_cap)) {
                        if (pos < 0 || pos >= idx_cap) r.bad_writes++;
                        else r.row[pos] = (int32_t)(t0 + th * kPer + i);
                    }
                    ++pos;
                }
        }
    }
    return r;
}

// The whole chain on consistent inputs.
static Result run_chain(const std::vector<uint32_t> &keys, int64_t L, int top_k, int n_init,
                        int n_local, int idx_cap) {
    const Windows w = windows(L, top_k, n_init, n_local);
    std::vector<uint32_t> hist(4 * 256, 0);
    auto cand = [&](int64_t t) { return t >= w.init_hi && t < w.local_lo; };
    uint32_t prefix = 0, mask = 0;
    int remaining = top_k;
    bool whole = false;
    if (w.choose) {
        for (int64_t t = 0; t < L; ++t)
            if (cand(t)) hist[keys[t] >> 24]++;
        for (int pass = 1; pass < 4; ++pass) {
            prefix_of(hist, pass, top_k, prefix, mask, remaining, whole);
            if (whole) break;
            const int shift = 24 - 8 * pass;
            for (int64_t t = 0; t < L; ++t)
                if (cand(t) && (keys[t] & mask) == prefix) hist[pass * 256 + ((keys[t] >> shift) & 255u)]++;
        }
        prefix_of(hist, 4, top_k, prefix, mask, remaining, whole);
    }
    const uint32_t thr = w.choose ? prefix : 0u;
    if (!w.choose) mask = 0xffffffffu;
    const int n_chunks = (int)((L + kChunk - 1) / kChunk);
    std::vector<int32_t> counts(2 * (n_chunks > 0 ? n_chunks : 1), 0);
    for (int64_t t = 0; t < L; ++t) {
        const int c = (int)(t / kChunk);
        if (!cand(t)) counts[2 * c]++;
        else if (w.take_all || (w.choose && (keys[t] & mask) > thr)) counts[2 * c]++;
        else if (w.choose && (keys[t] & mask) == thr) counts[2 * c + 1]++;
    }
    return write_row(keys, w, whole, counts, thr, (uint32_t)remaining, mask, idx_cap);
}

static std::vector<int32_t> brute(const std::vector<uint32_t> &keys, int64_t L, int top_k, int n_init,
                                  int n_local) {
    const Windows w = windows(L, top_k, n_init, n_local);
    std::vector<int32_t> out, c;
    for (int64_t t = 0; t < L; ++t) {
        if (t >= w.init_hi && t < w.local_lo) c.push_back((int32_t)t);
        else out.push_back((int32_t)t);
    }
    std::stable_sort(c.begin(), c.end(), [&](int32_t a, int32_t b) {
        return keys[a] > keys[b] || (keys[a] == keys[b] && a < b);
    });
    const int take = top_k < 0 ? 0 : (top_k < (int)c.size() ? top_k : (int)c.size());
    out.insert(out.end(), c.begin(), c.begin() + take);
    std::sort(out.begin(), out.end());
    return out;
}

int main() {
    std::mt19937_64 rng(12345);
    int fails = 0, cases = 0;
    // 1. consistent inputs, including many equal keys and short rows
    const int64_t lens[] = {0, 1, 100, 193, 4096, 4097, 9000, 12289};
    const int ks[] = {0, 1, 7, 64, 300, 5000};
    for (int64_t L : lens)
        for (int k : ks)
            for (int kind = 0; kind < 3; ++kind) {
                std::vector<uint32_t> keys(((L + kChunk - 1) / kChunk + 1) * kChunk);
                for (auto &x : keys) {
                    const uint64_t r = rng();
                    x = kind == 0 ? (uint32_t)r : (kind == 1 ? (uint32_t)(r % 5) << 24 | 0x800000u
                                                              : 0x80000000u | (uint32_t)(r % 3));
                }
                const int n_init = 16, n_local = 64;
                const int cap = k + n_init + n_local;
                const Result r = run_chain(keys, L, k, n_init, n_local, cap);
                const std::vector<int32_t> want = brute(keys, L, k, n_init, n_local);
                bool ok = r.bad_writes == 0 && r.cnt == (int)want.size();
                for (int i = 0; ok && i < cap; ++i)
                    ok = r.row[i] == (i < (int)want.size() ? want[i] : -1);
                ++cases;
                if (!ok) {
                    ++fails;
                    fprintf(stderr, "consistent case L=%ld k=%d kind=%d: cnt %d want %zu\n", (long)L, k,
                            kind, r.cnt, want.size());
                }
            }
    // 2. inconsistent inputs: random words everywhere the chain reads counts
    for (int trial = 0; trial < 400; ++trial) {
        const int64_t L = 1 + (int64_t)(rng() % 12000);
        const int k = (int)(rng() % 200);
        const int n_init = 4, n_local = 8;
        const int cap = k + n_init + n_local;
        const Windows w = windows(L, k, n_init, n_local);
        std::vector<uint32_t> keys(((L + kChunk - 1) / kChunk + 1) * kChunk);
        for (auto &x : keys) x = (uint32_t)rng();
        std::vector<uint32_t> hist(4 * 256);
        for (auto &h : hist) {
            const uint64_t r = rng();
            h = (r & 3) == 0 ? (uint32_t)(r >> 8) : (uint32_t)(r >> 40) % 64;   // some huge, some small
        }
        uint32_t prefix, mask;
        int remaining;
        bool whole;
        prefix_of(hist, 4, k, prefix, mask, remaining, whole);
        const int n_chunks = (int)((L + kChunk - 1) / kChunk);
        std::vector<int32_t> counts(2 * n_chunks);
        for (auto &c : counts) {
            const uint64_t r = rng();
            c = (r & 1) ? (int32_t)(uint32_t)(r >> 16) : (int32_t)((r >> 16) % 40) - 5;
        }
        const uint32_t take_word = (trial & 1) ? (uint32_t)rng() : (uint32_t)remaining;
        const Result r = write_row(keys, w, whole, counts, prefix, take_word, mask, cap);
        ++cases;
        if (r.bad_writes != 0 || r.cnt < 0 || r.cnt > cap) {
            ++fails;
            fprintf(stderr, "inconsistent trial %d: %ld bad writes, cnt %d cap %d\n", trial,
                    (long)r.bad_writes, r.cnt, cap);
        }
    }
    printf("%d cases, %d failures\n", cases, fails);
    return fails == 0 ? 0 : 1;
}
