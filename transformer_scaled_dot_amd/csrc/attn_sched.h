// Work lists of the persistent head_dim-128 attention kernel: which work items (256 query rows of one
// (batch, head)) each of its G workgroups runs, in order. Item index = query-block index * BH + bh, the
// query blocks in the schedule's order (the kernel maps block qt to rows (num_qtiles - 1 - qt) * 256 for
// the causal mask, so that the longest items come first). Plain integer code, compiled for the device by
// the kernel and for the host by the schedule's tests.
#pragma once

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#endif

#ifndef TSD_HD
#if defined(__HIPCC__)
#define TSD_HD __host__ __device__ __forceinline__
#else
#define TSD_HD inline
#endif
#endif

namespace tsd {

// Item of workgroup w in round k: even rounds in workgroup order, odd rounds reversed (by groups of 8 when
// G is a multiple of 8, so that the XCD stays the same).
TSD_HD int qb2_round_item(int w, int k, int G)
{
    const int i = (k & 1) ? ((G & 7) == 0 ? (G / 8 - 1 - w / 8) * 8 + (w & 7) : G - 1 - w) : w;
    return k * G + i;
}

// The j-th item workgroup w processes (>= num_items: none). A workgroup takes its rounds' items starting
// from round w mod (its item count), so that item boundaries -- where a workgroup waits for its next
// item's first tiles -- do not fall at the same time on every CU.
TSD_HD int qb2_sched(int w, int j, int G, int num_items)
{
    const int rounds = num_items / G;
    const int n_w = rounds + (qb2_round_item(w, rounds, G) < num_items ? 1 : 0);
    if (j >= n_w) return num_items;
    return qb2_round_item(w, (j + w) % n_w, G);
}

// Head-major alternative for grids of whole XCDs (G % 8 == 0, workgroup w on XCD w % 8) when every XCD can
// take the same number of whole rounds: XCD x runs the items of heads bh = x, x + 8, ... in head order, all
// query blocks of one head next to each other, so that the M = G / 8 workgroups of an XCD work on one or
// two heads at a time and share those heads' K/V tiles in the XCD's L2. Workgroup m takes slot m of even
// rounds and slot M - 1 - m of odd ones (long and short items alternate). Sets bh and the query-block
// index of the workgroup's j-th item (item index qt * BH + bh); false when it has none.
TSD_HD bool qb2_sched_heads(int w, int j, int G, int BH, int num_qtiles, int &bh, int &qt)
{
    const int M = G / 8, x = w & 7, m = w >> 3;
    const int rounds = (BH / 8) * num_qtiles / M;
    if (j >= rounds) return false;
    const int n = j * M + ((j & 1) ? M - 1 - m : m);
    const int k = n / num_qtiles;
    qt = n - k * num_qtiles;
    bh = x + 8 * k;
    return true;
}

TSD_HD bool qb2_heads_schedule(int G, int BH, int num_qtiles)
{
    return G % 8 == 0 && BH % 8 == 0 && ((BH / 8) * num_qtiles) % (G / 8) == 0;
}

}  // namespace tsd
