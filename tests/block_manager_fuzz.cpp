// Random-call driver for the host block manager (csrc/pool.cpp), built with
// g++ and AddressSanitizer + UndefinedBehaviorSanitizer by
// tests/test_host_sanitizers.py. Each round makes a pool of random geometry
// and issues random valid and invalid calls (extend, copy-on-write extend,
// fork, finish, trim, prefix register / acquire, alloc / free, garbage ids);
// after every call the free stack, the cached list and the reference counts
// must be consistent, and at the end every block must be back.
#include <cstdio>
#include <cstdlib>
#include <random>
#include <vector>
#include <algorithm>
#include "pagedkv.h"

static void check(pkv_pool* p, int nb) {
    // refcounts in range, free list consistent with refcount 0 (cached too)
    std::vector<int32_t> fl(nb + 1);
    int nf = kv_pool_free_list(p, fl.data(), nb + 1);
    std::vector<int32_t> cl(nb + 1);
    int nc = kv_pool_cached_list(p, cl.data(), nb + 1);
    if (nf < 0 || nc < 0 || nf + nc != kv_pool_num_free(p)) { printf("count mismatch\n"); abort(); }
    std::vector<int> seen(nb, 0);
    for (int i = 0; i < nf; ++i) { if (fl[i] < 0 || fl[i] >= nb || seen[fl[i]]++) { printf("bad free\n"); abort(); } if (block_refcount(p, fl[i]) != 0) abort(); }
    for (int i = 0; i < nc; ++i) { if (cl[i] < 0 || cl[i] >= nb || seen[cl[i]]++) { printf("bad cached\n"); abort(); } if (block_refcount(p, cl[i]) != 0) abort(); }
    for (int b = 0; b < nb; ++b) if (!seen[b] && block_refcount(p, b) <= 0) { printf("lost block %d\n", b); abort(); }
}

int main(int argc, char** argv) {
    const int iters = argc > 1 ? atoi(argv[1]) : 20000;
    std::mt19937_64 rng(12345);
    auto R = [&](int lo, int hi) { return (int)std::uniform_int_distribution<int>(lo, hi)(rng); };
    for (int round = 0; round < 40; ++round) {
        const int nb = R(1, 64), W = R(1, 10);
        pkv_pool_desc d{R(1, 3), nb, 16, R(1, 4), R(0, 1) ? 64 : 128, R(0, 2)};
        pkv_pool* p = nullptr;
        if (kv_pool_create(&d, nullptr, 0, &p) != PKV_OK) { printf("create failed %s\n", pkv_last_error()); return 1; }
        std::vector<std::vector<int32_t>> rows;
        std::vector<int32_t> lens;
        for (int it = 0; it < iters / 40; ++it) {
            const int op = R(0, 9);
            if (op == 0) {  // new sequence
                std::vector<int32_t> row(W, -1);
                int32_t cur = 0, nw = R(0, W * 16 + 3);
                std::vector<int64_t> slots(std::max(nw, 1));
                if (kv_seq_extend(p, 1, row.data(), W, &cur, &nw, slots.data()) == PKV_OK) { rows.push_back(row); lens.push_back(nw); }
            } else if (op == 1 && !rows.empty()) {  // grow all (cow)
                const int n = rows.size();
                std::vector<int32_t> flat(n * W), cur(lens), nw(lens);
                for (int i = 0; i < n; ++i) { std::copy(rows[i].begin(), rows[i].end(), flat.begin() + i * W); nw[i] = std::min(lens[i] + R(0, 3), W * 16 + R(0, 1)); }
                int64_t total = 0; for (int i = 0; i < n; ++i) total += std::max(0, nw[i] - cur[i]);
                std::vector<int64_t> slots(total + 1);
                std::vector<int32_t> cs(n + 1), cd(n + 1); int32_t nc = 0;
                if (kv_seq_extend_cow(p, n, flat.data(), W, cur.data(), nw.data(), slots.data(), cs.data(), cd.data(), &nc) == PKV_OK) {
                    for (int i = 0; i < n; ++i) { std::copy(flat.begin() + i * W, flat.begin() + (i + 1) * W, rows[i].begin()); lens[i] = nw[i]; }
                }
            } else if (op == 2 && !rows.empty()) {  // finish
                const int i = R(0, rows.size() - 1);
                std::vector<int32_t> ids;
                for (int j = 0; j < (lens[i] + 15) / 16 && j < W; ++j) if (rows[i][j] >= 0) ids.push_back(rows[i][j]);
                if (block_free(p, ids.size(), ids.data()) != PKV_OK) { printf("free failed %s\n", pkv_last_error()); abort(); }
                rows.erase(rows.begin() + i); lens.erase(lens.begin() + i);
            } else if (op == 3 && !rows.empty()) {  // fork
                const int i = R(0, rows.size() - 1);
                const int nbk = (lens[i] + 15) / 16;
                bool ok = true; for (int j = 0; j < nbk; ++j) ok &= rows[i][j] >= 0;
                std::vector<int32_t> dst(W, -1);
                if (ok && kv_seq_fork(p, rows[i].data(), dst.data(), nbk) == PKV_OK) { rows.push_back(dst); lens.push_back(lens[i]); }
            } else if (op == 4 && !rows.empty()) {  // trim
                const int n = rows.size();
                std::vector<int32_t> flat(n * W);
                for (int i = 0; i < n; ++i) std::copy(rows[i].begin(), rows[i].end(), flat.begin() + i * W);
                int32_t rel = 0;
                if (kv_seq_trim(p, n, flat.data(), W, lens.data(), R(1, 60), &rel) == PKV_OK)
                    for (int i = 0; i < n; ++i) std::copy(flat.begin() + i * W, flat.begin() + (i + 1) * W, rows[i].begin());
            } else if (op == 5 && !rows.empty()) {  // register keys
                const int i = R(0, rows.size() - 1);
                std::vector<uint64_t> keys; std::vector<int32_t> ids;
                for (int j = 0; j < lens[i] / 16 && j < W; ++j) if (rows[i][j] >= 0) { keys.push_back((uint64_t)R(1, 40)); ids.push_back(rows[i][j]); }
                int32_t taken = 0;
                kv_prefix_register(p, keys.data(), ids.data(), ids.size(), &taken);
            } else if (op == 6) {  // acquire and release
                std::vector<uint64_t> keys(R(0, 5)); for (auto& k : keys) k = (uint64_t)R(1, 40);
                std::vector<int32_t> ids(keys.size() + 1); int32_t m = 0;
                if (kv_prefix_acquire(p, keys.data(), keys.size(), ids.data(), &m) == PKV_OK && m > 0)
                    if (block_free(p, m, ids.data()) != PKV_OK) abort();
            } else if (op == 7) {  // garbage calls that must fail cleanly
                int32_t bad[4] = {-7, nb, nb + 100, (int32_t)0x7fffffff};
                block_free(p, 4, bad); block_incref(p, 4, bad);
                int32_t out[8]; block_alloc(p, -3, out); block_alloc(p, nb + 5, out);
                int32_t cur = 5, nw = 3; int64_t s[4]; std::vector<int32_t> row(W, -1);
                kv_seq_extend(p, 1, row.data(), W, &cur, &nw, s);
                int32_t rel; kv_seq_trim(p, 1, row.data(), W, &cur, 0, &rel);
                kv_seq_trim(nullptr, 1, row.data(), W, &cur, 4, &rel);
                kv_seq_fork(p, bad, row.data(), 3);
            } else if (op == 8) {  // alloc/free churn
                int32_t out[8]; const int k = R(0, 8);
                if (block_alloc(p, k, out) == PKV_OK && block_free(p, k, out) != PKV_OK) abort();
            } else if (op == 9 && !rows.empty()) {  // shared extend (no cow) must refuse appending into shared blocks
                const int i = R(0, rows.size() - 1);
                int32_t cur = lens[i], nw = std::min(lens[i] + 1, W * 16); int64_t s[2];
                std::vector<int32_t> row = rows[i];
                if (kv_seq_extend(p, 1, row.data(), W, &cur, &nw, s) == PKV_OK) { rows[i] = row; lens[i] = nw; }
            }
            check(p, nb);
        }
        for (size_t i = 0; i < rows.size(); ++i) {
            std::vector<int32_t> ids;
            for (int j = 0; j < (lens[i] + 15) / 16 && j < W; ++j) if (rows[i][j] >= 0) ids.push_back(rows[i][j]);
            if (block_free(p, ids.size(), ids.data()) != PKV_OK) { printf("final free failed %s\n", pkv_last_error()); abort(); }
        }
        if (kv_pool_num_free(p) != nb) { printf("leak: %d of %d free\n", kv_pool_num_free(p), nb); abort(); }
        kv_pool_destroy(p);
    }
    printf("ok\n");
    return 0;
}
