// K-tail kernels of table row 2 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW_TAIL(2, Fast2)
