// K-tail kernels of table row 9 (see mg_table.h).
#include "mg_launch.h"

MG_DEFINE_ROW_TAIL(9, Fast9)
