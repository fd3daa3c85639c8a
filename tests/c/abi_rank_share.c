/*
 * A plain C consumer of libspattn.so: one rank's share of packed-token
 * sequence-parallel attention driven through the C ABI alone (no Python, no
 * torch), as a host program of the library would.
 *
 *   abi_rank_share IN OUT
 *
 * IN:  int64 S, W, r, H, d, then the bf16 bit patterns of Q, K and V of the
 *      whole sequence, each [S, H, d].
 * OUT: rank r's output O [s_r, H, d] as bf16 bit patterns, then its LSE
 *      [H, s_r] as float32.
 *
 * Steps (page "HCCL AllGatherV 实战解析：MiniMax-H3-Comfy-NPU ...", sections
 * 机制一 and 后端 A): shard bounds; RoPE of every rank's K slice and of rank
 * r's Q slice at absolute positions; AllGatherV of the K and V shards (pack
 * into one flat buffer, then unpack); attention of the local queries against
 * the full K/V.  It also checks one error path (overlapping displacements).
 * Exit status 0 on success; every failing call prints sp_last_error().
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "spattn.h"

#define MAXW 16

static int hip_ok(hipError_t e, const char* what) {
  if (e != hipSuccess) {
    fprintf(stderr, "%s: %s\n", what, hipGetErrorString(e));
    return 0;
  }
  return 1;
}

static int sp_ok(int st, const char* what) {
  if (st != SP_OK) {
    fprintf(stderr, "%s: status %d: %s\n", what, st, sp_last_error());
    return 0;
  }
  return 1;
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  FILE* f = fopen(argv[1], "rb");
  if (!f) { perror(argv[1]); return 2; }
  int64_t hdr[5];
  if (fread(hdr, sizeof(int64_t), 5, f) != 5) { fprintf(stderr, "short header\n"); fclose(f); return 2; }
  const int64_t S = hdr[0];
  const int32_t W = (int32_t)hdr[1], r = (int32_t)hdr[2], H = (int32_t)hdr[3], d = (int32_t)hdr[4];
  if (S < 1 || W < 1 || W > MAXW || r < 0 || r >= W || H < 1 || d < 1) { fprintf(stderr, "bad header\n"); fclose(f); return 2; }
  const int64_t inner = (int64_t)H * d, n = S * inner;
  uint16_t* host = (uint16_t*)malloc((size_t)(3 * n) * sizeof(uint16_t));
  if (!host || fread(host, sizeof(uint16_t), (size_t)(3 * n), f) != (size_t)(3 * n)) {
    fprintf(stderr, "short input\n");
    fclose(f);
    free(host);
    return 2;
  }
  fclose(f);
  const uint16_t *hq = host, *hk = host + n, *hv = host + 2 * n;

  int64_t lo[MAXW], hi[MAXW], lens[MAXW], counts[MAXW], displs[MAXW];
  for (int32_t i = 0; i < W; ++i) {
    if (!sp_ok(sp_shard_bounds(S, W, i, &lo[i], &hi[i]), "sp_shard_bounds")) return 1;
    lens[i] = hi[i] - lo[i];
  }
  if (!sp_ok(sp_allgatherv_layout(S, W, 1, inner, counts, displs), "sp_allgatherv_layout")) return 1;
  const int64_t sq = lens[r];

  hipStream_t stream;
  if (!hip_ok(hipStreamCreate(&stream), "hipStreamCreate")) return 1;
  void *dk, *dv, *dq, *flat_k, *flat_v, *k_full, *v_full, *dout;
  float* dlse;
  const size_t nb = (size_t)n * 2, qb = (size_t)(sq * inner) * 2;
  if (!hip_ok(hipMalloc(&dk, nb), "hipMalloc") || !hip_ok(hipMalloc(&dv, nb), "hipMalloc") ||
      !hip_ok(hipMalloc(&dq, qb), "hipMalloc") || !hip_ok(hipMalloc(&flat_k, nb), "hipMalloc") ||
      !hip_ok(hipMalloc(&flat_v, nb), "hipMalloc") || !hip_ok(hipMalloc(&k_full, nb), "hipMalloc") ||
      !hip_ok(hipMalloc(&v_full, nb), "hipMalloc") || !hip_ok(hipMalloc(&dout, qb), "hipMalloc") ||
      !hip_ok(hipMalloc((void**)&dlse, (size_t)(H * sq) * sizeof(float)), "hipMalloc"))
    return 1;
  /* every rank's K and V slice, side by side in one buffer each (the "send" shards) */
  if (!hip_ok(hipMemcpy(dk, hk, nb, hipMemcpyHostToDevice), "hipMemcpy") ||
      !hip_ok(hipMemcpy(dv, hv, nb, hipMemcpyHostToDevice), "hipMemcpy") ||
      !hip_ok(hipMemcpy(dq, hq + lo[r] * inner, qb, hipMemcpyHostToDevice), "hipMemcpy"))
    return 1;

  const void* ksend[MAXW];
  const void* vsend[MAXW];
  for (int32_t i = 0; i < W; ++i) {
    void* ki = (char*)dk + lo[i] * inner * 2;
    ksend[i] = ki;
    vsend[i] = (const char*)dv + lo[i] * inner * 2;
    /* each rank rotates its own K slice in place, at absolute positions */
    if (!sp_ok(rope_apply(SP_BF16, ki, ki, lens[i], H, d, lo[i], 10000.0, SP_ROPE_HALF, stream), "rope_apply K"))
      return 1;
  }
  if (!sp_ok(rope_apply(SP_BF16, dq, dq, sq, H, d, lo[r], 10000.0, SP_ROPE_HALF, stream), "rope_apply Q") ||
      !sp_ok(varlen_pack(SP_BF16, W, ksend, counts, displs, flat_k, n, stream), "varlen_pack K") ||
      !sp_ok(varlen_pack(SP_BF16, W, vsend, counts, displs, flat_v, n, stream), "varlen_pack V") ||
      !sp_ok(varlen_unpack(SP_BF16, W, flat_k, n, displs, lens, 1, inner, k_full, stream), "varlen_unpack K") ||
      !sp_ok(varlen_unpack(SP_BF16, W, flat_v, n, displs, lens, 1, inner, v_full, stream), "varlen_unpack V") ||
      !sp_ok(shard_attn_fwd(SP_BF16, dq, k_full, v_full, dout, dlse, sq, S, H, d, (float)(1.0 / sqrt((double)d)),
                            stream), "shard_attn_fwd"))
    return 1;

  /* error path: two ranks' blocks overlap in the flat buffer -> rejected, nothing enqueued */
  int64_t bad[MAXW];
  memcpy(bad, displs, sizeof(bad));
  if (W > 1) {
    bad[1] = displs[0] + (counts[0] > 0 ? 1 : 0);
    const int st = varlen_pack(SP_BF16, W, ksend, counts, bad, flat_k, n, stream);
    printf("error path: status %d: %s\n", st, sp_last_error());
    if (counts[0] > 1 && counts[1] > 0 && st != SP_EOVERLAP) { fprintf(stderr, "overlap not rejected\n"); return 1; }
  }

  if (!hip_ok(hipStreamSynchronize(stream), "hipStreamSynchronize")) return 1;
  uint16_t* ho = (uint16_t*)malloc(qb);
  float* hl = (float*)malloc((size_t)(H * sq) * sizeof(float));
  if (!ho || !hl) return 1;
  if (!hip_ok(hipMemcpy(ho, dout, qb, hipMemcpyDeviceToHost), "hipMemcpy") ||
      !hip_ok(hipMemcpy(hl, dlse, (size_t)(H * sq) * sizeof(float), hipMemcpyDeviceToHost), "hipMemcpy"))
    return 1;
  FILE* g = fopen(argv[2], "wb");
  if (!g) { perror(argv[2]); return 2; }
  const int wrote = fwrite(ho, 2, (size_t)(sq * inner), g) == (size_t)(sq * inner) &&
                    fwrite(hl, sizeof(float), (size_t)(H * sq), g) == (size_t)(H * sq);
  fclose(g);
  if (!wrote) { fprintf(stderr, "short write\n"); return 2; }
  printf("rank %d of %d: %lld queries x %d heads x %d against %lld keys, ABI version %d\n", r, W, (long long)sq, H, d,
         (long long)S, sp_abi_version());

  hipFree(dk); hipFree(dv); hipFree(dq); hipFree(flat_k); hipFree(flat_v);
  hipFree(k_full); hipFree(v_full); hipFree(dout); hipFree(dlse);
  hipStreamDestroy(stream);
  free(host); free(ho); free(hl);
  return 0;
}
