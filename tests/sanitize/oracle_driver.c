/*
 * oracle_driver.c -- runs the fp64 oracle (oracle/gdn_oracle.c, compiled into
 * this program) under AddressSanitizer and UndefinedBehaviorSanitizer on the
 * CPU.  TEST INFRASTRUCTURE ONLY.
 *
 * Input file (little-endian): int64 N, H, dk, dv, tokens, has_h0, has_dht,
 * nthreads; double scale; int64 cu[N+1]; double q, k [tokens][H][dk],
 * v [tokens][H][dv], g, beta [tokens][H], h0 [N][H][dk][dv] (if has_h0),
 * do [tokens][H][dv], dht [N][H][dk][dv] (if has_dht).
 * Output file: o, ht, dq, dk, dv, dg, dbeta, dh0 in that order (doubles).
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

int gdn_oracle_fwd(int64_t nseq, const int64_t* cu, int64_t H, int64_t dk, int64_t dv, double scale,
                   const double* q, const double* k, const double* v, const double* g, const double* beta,
                   const double* h0, double* o, double* ht, int nthreads);
int gdn_oracle_bwd(int64_t nseq, const int64_t* cu, int64_t H, int64_t dk, int64_t dv, double scale,
                   const double* q, const double* k, const double* v, const double* g, const double* beta,
                   const double* h0, const double* dO, const double* dht, double* dq, double* dk_, double* dv_,
                   double* dg, double* dbeta, double* dh0, int nthreads);

static void* take(FILE* f, size_t n, size_t sz) {
  void* p = malloc(n * sz ? n * sz : 1);
  if (!p || fread(p, sz, n, f) != n) {
    fprintf(stderr, "short input\n");
    exit(2);
  }
  return p;
}

int main(int argc, char** argv) {
  if (argc != 3) return 2;
  FILE* f = fopen(argv[1], "rb");
  if (!f) return 2;
  int64_t hd[8];
  if (fread(hd, sizeof(int64_t), 8, f) != 8) return 2;
  const int64_t N = hd[0], H = hd[1], dk = hd[2], dv = hd[3], T = hd[4];
  double scale;
  if (fread(&scale, sizeof(double), 1, f) != 1) return 2;
  int64_t* cu = take(f, (size_t)(N + 1), sizeof(int64_t));
  double* q = take(f, (size_t)(T * H * dk), sizeof(double));
  double* k = take(f, (size_t)(T * H * dk), sizeof(double));
  double* v = take(f, (size_t)(T * H * dv), sizeof(double));
  double* g = take(f, (size_t)(T * H), sizeof(double));
  double* beta = take(f, (size_t)(T * H), sizeof(double));
  double* h0 = hd[5] ? take(f, (size_t)(N * H * dk * dv), sizeof(double)) : NULL;
  double* dO = take(f, (size_t)(T * H * dv), sizeof(double));
  double* dht = hd[6] ? take(f, (size_t)(N * H * dk * dv), sizeof(double)) : NULL;
  fclose(f);
  const size_t so = (size_t)(T * H * dv), ss = (size_t)(N * H * dk * dv);
  double* o = calloc(so ? so : 1, sizeof(double));
  double* ht = calloc(ss ? ss : 1, sizeof(double));
  double* dq = calloc((size_t)(T * H * dk) + 1, sizeof(double));
  double* dk_ = calloc((size_t)(T * H * dk) + 1, sizeof(double));
  double* dv_ = calloc(so + 1, sizeof(double));
  double* dg = calloc((size_t)(T * H) + 1, sizeof(double));
  double* db = calloc((size_t)(T * H) + 1, sizeof(double));
  double* dh0 = calloc(ss + 1, sizeof(double));
  if (gdn_oracle_fwd(N, cu, H, dk, dv, scale, q, k, v, g, beta, h0, o, ht, (int)hd[7])) return 3;
  if (gdn_oracle_bwd(N, cu, H, dk, dv, scale, q, k, v, g, beta, h0, dO, dht, dq, dk_, dv_, dg, db, dh0, (int)hd[7]))
    return 4;
  FILE* out = fopen(argv[2], "wb");
  if (!out) return 2;
  fwrite(o, sizeof(double), so, out);
  fwrite(ht, sizeof(double), ss, out);
  fwrite(dq, sizeof(double), (size_t)(T * H * dk), out);
  fwrite(dk_, sizeof(double), (size_t)(T * H * dk), out);
  fwrite(dv_, sizeof(double), so, out);
  fwrite(dg, sizeof(double), (size_t)(T * H), out);
  fwrite(db, sizeof(double), (size_t)(T * H), out);
  fwrite(dh0, sizeof(double), ss, out);
  fclose(out);
  free(cu); free(q); free(k); free(v); free(g); free(beta); free(h0); free(dO); free(dht);
  free(o); free(ht); free(dq); free(dk_); free(dv_); free(dg); free(db); free(dh0);
  printf("ok\n");
  return 0;
}
