/* A plain C (and C++) caller of the boundary: includes mb.h, links libmb.so
 * and exercises the calls that need no GPU (version, status names, argument
 * validation that returns before any HIP call). */
#include "mb.h"

#include <stdio.h>

int main(void) {
  int bad = 0;
  printf("abi %d\n", mb_abi_version());
  printf("%s\n", mb_status_string(MB_ERR_SHAPE));
  /* required pointers missing */
  bad |= mb_bias_gelu_fwd(NULL, NULL, NULL, 4, 8, MB_BF16, (hipStream_t)0) != MB_ERR_NULL;
  /* a row that is not whole 16-byte vectors */
  bad |= mb_bias_gelu_fwd((const void*)16, NULL, (void*)4096, 4, 7, MB_BF16, (hipStream_t)0) != MB_ERR_SHAPE;
  /* probability outside [0, 1] */
  bad |= mb_bias_dropout_add_train((const void*)16, NULL, (const void*)4096, MB_BF16, (void*)8192, 4, 8, MB_BF16,
                                   1.5f, 1234u, 0u, (hipStream_t)0) != MB_ERR_PROB;
  /* workspace queries are pure host arithmetic */
  bad |= mb_bias_gelu_bwd_workspace(16384, 32768, MB_BF16, 1) == 0;
  bad |= mb_bias_gelu_bwd_workspace(16384, 32768, MB_BF16, 0) != 0;
  printf("%s\n", bad ? "FAIL" : "ok");
  return bad;
}
