/* Prints the cache element offsets the public header's inline helpers give,
 * for a caller that fills a paged cache without pkv_append.  Reads lines of
 * "num_blocks num_kv_heads block_size head_dim dtype block head t d" from
 * stdin and writes "k_offset v_offset" per line.  Built and run by the CPU
 * layout test; it links nothing but the header. */
#include <stdio.h>

#include "pkv.h"

int main(void)
{
    pkv_cache_desc c;
    int blk, head, t, d;
    while (scanf("%d %d %d %d %d %d %d %d %d", &c.num_blocks, &c.num_kv_heads, &c.block_size,
                 &c.head_dim, &c.dtype, &blk, &head, &t, &d) == 9)
        printf("%lld %lld\n", (long long)pkv_k_elem_offset(&c, blk, head, t, d),
               (long long)pkv_v_elem_offset(&c, blk, head, t, d));
    return 0;
}
