/* Host-side checks of the C ABI's validation paths under AddressSanitizer:
 * every call here is rejected (or only sizes a workspace) before any launch. */
#include <stdio.h>
#include <stdlib.h>
#include "gsq.h"

#define EXPECT(c) do { if (!(c)) { printf("FAIL %s:%d %s\n", __FILE__, __LINE__, #c); return 1; } } while (0)

int main(void) {
    for (int s = -2; s < 10; ++s) EXPECT(gsq_status_str(s) != NULL);
    for (int g = -1; g < 6; ++g) (void)gsq_num_logits(g);
    /* host token-offset arrays sized exactly E + 1 on the heap */
    int64_t* offs = malloc(sizeof(int64_t) * 4);
    offs[0] = 0; offs[1] = 128; offs[2] = 128; offs[3] = 320;
    EXPECT(gsq_recon_workspace_bytes(3, offs, 256, 256) > 0);
    offs[2] = 64;   /* decreasing: rejected */
    EXPECT(gsq_recon_workspace_bytes(3, offs, 256, 256) == 0);
    offs[2] = 128; offs[3] = 130;   /* not a multiple of 64 */
    EXPECT(gsq_recon_workspace_bytes(3, offs, 256, 256) == 0);
    free(offs);
    int64_t* one = malloc(sizeof(int64_t) * 2);
    one[0] = 0; one[1] = 4096;
    EXPECT(gsq_recon_workspace_bytes(1, one, 5000, 4096) == (size_t)((384 * 4 + 255) / 256 * 256 + 256));
    EXPECT(gsq_recon_workspace_bytes(0, one, 5000, 4096) == 0);
    EXPECT(gsq_recon_workspace_bytes(1, NULL, 5000, 4096) == 0);
    /* recon call rejected on a NULL device pointer after reading the offsets */
    EXPECT(gsq_recon_loss_grad(1, one, 64, 256, NULL, NULL, NULL, NULL, 0, NULL, NULL, NULL, NULL) != GSQ_OK);
    free(one);
    EXPECT(gsq_recon_gram_workspace_bytes(5000, 4096) > 0);
    EXPECT(gsq_recon_gram_workspace_bytes(5000, 100) == 0);
    EXPECT(gsq_gptq_workspace_bytes(64, 256) > 0);
    EXPECT(gsq_gptq_workspace_bytes(64, 100) == 0);
    gsq_layer* lay = malloc(sizeof(gsq_layer));
    lay->grid = GSQ_GRID_INT2; lay->group = 128; lay->rows = 4; lay->cols = 256;
    lay->w_dtype = GSQ_DTYPE_BF16; lay->stream = 0; lay->seed = 1;
    EXPECT(gsq_relax_fwd(NULL, NULL, NULL, NULL, NULL, 0, 1.0f, 1.0f, NULL, NULL, NULL) == GSQ_ERR_NULL);
    EXPECT(gsq_relax_fwd(lay, NULL, NULL, NULL, NULL, 0, 1.0f, 1.0f, NULL, NULL, NULL) == GSQ_ERR_NULL);
    lay->grid = 9;
    EXPECT(gsq_relax_fwd(lay, (float*)0x10000, (float*)0x10000, NULL, (void*)0x10000, 0, 1.0f, 1.0f,
                         (uint16_t*)0x10000, NULL, NULL) == GSQ_ERR_GRID);
    free(lay);
    printf("asan driver ok\n");
    return 0;
}
